// Wave-index decode step on gfx950: score -> select + estimate -> exact attention -> LSE merge.
//
// Method: RetroInfer's tripartite attention (technical summary, gist.science Spanish page,
// section 2.A items 1-3; Arabic page section 2.a).  Per query head, the steady zone (sinks and
// local window) and the retrieval zone (all tokens of the top_k clusters by <q, mu_c>) are
// attended exactly; every other non-empty cluster contributes n_c * exp(s_c) to the softmax
// denominator and n_c * exp(s_c) * SV_c / n_c to the numerator; the partial softmax states are
// merged with log-sum-exp.
//
// The estimation is computed over *all* non-empty clusters, before the selection is known, and
// the terms of the retrieved clusters are subtracted at the merge: sum over E = sum over all -
// sum over R.  The subtracted terms never exceed the exact mass of the same tokens (exp is
// convex, so n_c exp(mean logit) is at most the sum of the members' exp(logit)), so the
// cancellation costs O(eps_fp32) relative to the merged denominator.  When a head retrieves every
// non-empty cluster both terms are dropped.
//
// Kernels (one stream, in order):
//   k_score      grid (ceil(C/128), B*Hkv): MFMA scores of the KV group's query heads against 128
//                centroids (one pass over mu serves all heads of the group), the score keys, the
//                tile's 8 best keys per head, fp32 centroid norms and non-empty counts.
//   k_select     grid (B*Hkv*E + B*Hq): the first B*Hkv*E workgroups stream the value sums and
//                fold the estimation partials (E per KV group); workgroup B*Hkv*E + bh finds the
//                exact top-k of query head bh (a threshold bounded from the tile summaries and found on the fp32
//                scores, canonical fp64 re-scoring of the certified uncertainty band, ties to the
//                lower id), published as the head's ascending list of clusters with their first
//                rows and token offsets.
//   k_attend     grid (B*Hq * (S + Sc)): S workgroups per head split its token list (steady zone,
//                then the rows of its retrieved clusters) with an online softmax; Sc workgroups
//                fold the retrieved clusters' estimation terms.
//   k_merge      grid (B*Hq): log-sum-exp merge of the head's partials into out and lse.
#include "wi_device.h"
#include "wi_internal.h"

namespace wi {

constexpr int kScoreThreads = 256;

// Workgroups of the attention and merge launches are numbered group-fastest: workgroup j serves
// query head (j mod BG) G + j / BG, so that consecutive numbers cycle through the KV groups.
// Workgroups are dispatched to the XCDs round-robin, so with BG a multiple of the 8 XCDs a
// group's attention workgroups and the merge of its heads share an XCD (and its L2).
__device__ __forceinline__ int head_of_block(const DecodeArgs& a, int j) {
  const int BG = a.B * a.Hkv, bg = j % BG;
  return bg * a.G + j / BG;
}

// ============================================================================ k_score
// grid (ceil(C/128), B*Hkv), 256 threads.  bf16: each wave copies its 32 centroid rows from HBM
// into LDS with direct global-to-LDS loads, one kilobyte (four whole rows) per instruction, and
// reads them back in the MFMA operand layout; a row's sixteen 16-byte pieces are stored rotated
// by an XOR with the row index, so that the 16 lanes of a read phase hit 16 different bank
// groups.  fp32: a centroid row (512 B) is read straight into the operand registers, as eight
// 64-byte pieces of 16 rows per instruction.  Centroid rows are read once per step, so both
// forms load them non-temporally (1M tokens: 29.2 -> 27.8 us; batch 16: 53.1 -> 51.2 us).  Four
// waves per SIMD where the tile's registers fit in 128 VGPRs without spilling (bf16, up to four
// heads per group); otherwise the compiler's choice.
template <typename T, int G> struct ScoreWaves { static constexpr int v = (sizeof(T) == 2 && G <= 4) ? 4 : 1; };

template <typename T, int G>
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(ScoreWaves<T, G>::v))) void k_score(DecodeArgs a) {
  constexpr bool kBf = sizeof(T) == 2;
  // fp32: per cluster of the tile its size (0 past nrows), its centroid's norm and the order keys
  // of its raw scores.  bf16: the tile's centroid rows, 16 pieces of 16 B per row, piece c of row
  // r at r * 16 + (c ^ (r & 15)); once a wave holds its 32 rows in registers, the same three
  // per-cluster values of its clusters go into the first 1280 bytes of its 8 KB of rows, so that
  // a workgroup needs 32 KB of LDS and five fit one CU.
  __shared__ float sh_n[kBf ? 1 : kScoreThreads];
  __shared__ float sh_nrm[kBf ? 1 : kScoreTile];
  __shared__ uint32_t sh_k[kBf ? 1 : G][kBf ? 1 : kScoreTile];
  __shared__ __attribute__((aligned(16))) u32x4_t sh_mu[kBf ? kScoreTile * 16 : 1];
  auto wreg = [&](int c) -> uint32_t* { return reinterpret_cast<uint32_t*>(sh_mu + (c >> 5) * 32 * 16); };
  auto key_at = [&](int h, int c) -> uint32_t& { if constexpr (kBf) return wreg(c)[h * 32 + (c & 31)]; else return sh_k[h][c]; };
  auto nrm_at = [&](int c) -> float& { if constexpr (kBf) return reinterpret_cast<float*>(wreg(c))[256 + (c & 31)]; else return sh_nrm[c]; };
  auto n_at = [&](int c) -> float& { if constexpr (kBf) return reinterpret_cast<float*>(wreg(c))[288 + (c & 31)]; else return sh_n[c]; };
  const int tile = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int C = a.C;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  if (C == 0) return;
  const int nrows = min(kScoreTile, C - tile * kScoreTile);
  const int cbase = tile * kScoreTile + w * 32;
  const T* mu = static_cast<const T*>(a.mu) + (size_t)bg * C * kD;
  const int32_t* szs = a.sizes + (size_t)bg * C;
  const T* qg = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)g * G) * kD;

  // Every global load of the tile is issued before the first wait: the sizes, the centroids and
  // the queries.  The loads are unconditional (row indices clamped into the tile, query rows
  // into the group) so that the wait before the first MFMA counts only the loads issued ahead
  // of it; query rows past the group are never read back.  Empty clusters are masked by their
  // size in the per-head pass.
  // the size of cluster ncl: bf16, lane l < 32 of wave w takes cluster 32 w + l (its wave's own
  // clusters); fp32, thread t takes cluster t
  const int ncl = kBf ? w * 32 + (lane & 31) : tid;
  const int n_raw = szs[tile * kScoreTile + min(ncl, nrows - 1)];
  // raw score of query head h (row h of the MFMA tile) against cluster row cl, and the norm of
  // that centroid
  auto put_scores = [&](const f32x4_t& acc, float n2, int t) {
    const int cl = w * 32 + 16 * t + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * lg + r;
      if (h < G) key_at(h, cl) = f32_order_key(acc[r]);
    }
    if (lg == 0) nrm_at(cl) = sqrtf(n2);
  };

  if constexpr (sizeof(T) == 2) {
    // A = query heads (row = lane&15), B = centroids (column = lane&15).  MFMA step s consumes
    // dims 32 s + 8 lg .. +8 on both operands, so the four lanes of a row read 64 contiguous bytes.
    bf16x8_t qa[4];
    bf16x8_t mb[2][4];
    // load i of the wave copies rows 4 i .. 4 i + 3 of its 32 (clamped into the group's rows):
    // lane L reads piece (L & 15) ^ (r & 15) of row r = 4 i + (L >> 4), which lands in LDS slot
    // L of the load's 64
    u32x4_t* wrows = sh_mu + w * 32 * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rl = 4 * i + (lane >> 4);                 // row within the wave's 32
      const int r = min(cbase + rl, C - 1);
      const int c = (lane & 15) ^ (rl & 15);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4_t*>(mu + (size_t)r * kD) + c,
                                       (__attribute__((address_space(3))) void*)(wrows + 64 * i), 16, 0, 2);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qa[s] = *reinterpret_cast<const bf16x8_t*>(qg + (size_t)min(lr, G - 1) * kD + 32 * s + 8 * lg);
    // the wave's own rows have landed in LDS (no other wave reads them)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rl = 16 * t + lr;
#pragma unroll
      for (int s = 0; s < 4; ++s) mb[t][s] = __builtin_bit_cast(bf16x8_t, wrows[rl * 16 + ((4 * s + lg) ^ (rl & 15))]);
    }
    // every row is in registers before the wave writes its per-cluster values over them
    __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], mb[t][s], acc, 0, 0, 0);
      float n2 = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float x = (float)mb[t][s][e]; n2 += x * x; }
      n2 += __shfl_xor(n2, 16);
      n2 += __shfl_xor(n2, 32);
      put_scores(acc, n2, t);
    }
  } else {
    // fp32: 16x16x4 MFMA, 32 steps; lane (lr, lg) loads dims 16 j + 4 lg .. +4 (j = 0..7) and step
    // 4 j + e consumes dim 16 j + 4 lg + e on both operands.
    u32x4_t mraw[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float* row = reinterpret_cast<const float*>(mu) + (size_t)min(cbase + 16 * t + lr, C - 1) * kD + 4 * lg;
#pragma unroll
      for (int j = 0; j < 8; ++j) mraw[t][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + 16 * j));
    }
    float qa[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const float*>(qg) + (size_t)min(lr, G - 1) * kD + 16 * j + 4 * lg);
      qa[4 * j] = __uint_as_float(v.x); qa[4 * j + 1] = __uint_as_float(v.y);
      qa[4 * j + 2] = __uint_as_float(v.z); qa[4 * j + 3] = __uint_as_float(v.w);
    }
    __builtin_amdgcn_sched_barrier(0);      // every load is in flight before the first wait
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float mb[32];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mb[4 * j] = __uint_as_float(mraw[t][j].x); mb[4 * j + 1] = __uint_as_float(mraw[t][j].y);
        mb[4 * j + 2] = __uint_as_float(mraw[t][j].z); mb[4 * j + 3] = __uint_as_float(mraw[t][j].w);
      }
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 32; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[s], mb[s], acc, 0, 0, 0);
      float n2 = 0.f;
#pragma unroll
      for (int s = 0; s < 32; ++s) n2 += mb[s] * mb[s];
      n2 += __shfl_xor(n2, 16);
      n2 += __shfl_xor(n2, 32);
      put_scores(acc, n2, t);
    }
  }
  if (!kBf || lane < 32) n_at(ncl) = ncl < nrows ? (float)n_raw : 0.f;
  __syncthreads();

  const size_t slot = (size_t)bg * a.tiles_g + tile;
  if (w == 0) {
    // largest norm among the tile's non-empty centroids, and how many are non-empty
    const bool e0 = n_at(lane) > 0.f, e1 = n_at(lane + 64) > 0.f;
    const float nm = wave_max(fmaxf(e0 ? nrm_at(lane) : 0.f, e1 ? nrm_at(lane + 64) : 0.f));
    const int nc = __popcll(__ballot(e0)) + __popcll(__ballot(e1));
    if (lane == 0) { a.tile_norm[slot] = nm; a.tile_cnt[slot] = nc; }
  }
  // per head: the raw-score keys (0 for empty clusters) and the head's 8 best scores of the tile
  // (key 0 past the non-empty clusters) with their cluster ids: lane r keeps the r-th, found by
  // repeated wave maxima, each time clearing the holder with the lowest id
  for (int h = w; h < G; h += kScoreThreads / 64) {
    const bool e0 = n_at(lane) > 0.f, e1 = n_at(lane + 64) > 0.f;
    const uint32_t k0 = e0 ? key_at(h, lane) : 0u, k1 = e1 ? key_at(h, lane + 64) : 0u;
    uint32_t* keys_h = a.keys + ((size_t)b * a.Hq + (size_t)g * G + h) * C + (size_t)tile * kScoreTile;
    if (lane < nrows) keys_h[lane] = k0;
    if (lane + 64 < nrows) keys_h[lane + 64] = k1;
    uint32_t c0 = k0, c1 = k1, best = 0u;
    int best_id = 0;
#pragma unroll
    for (int r = 0; r < kTileTop; ++r) {
      const uint32_t m8 = wave_umax(c0 > c1 ? c0 : c1);
      const uint64_t b0 = __ballot(c0 == m8);
      int holder;
      if (b0 != 0ull) {
        holder = __ffsll((unsigned long long)b0) - 1;
        if (lane == holder) c0 = 0u;
      } else {
        const uint64_t b1 = __ballot(c1 == m8);
        holder = __ffsll((unsigned long long)b1) - 1 + 64;
        if (lane == holder - 64) c1 = 0u;
      }
      if (lane == r) { best = m8; best_id = tile * kScoreTile + holder; }
    }
    if (lane < kTileTop) {
      const size_t ti = (((size_t)b * a.Hq + (size_t)g * G + h) * a.tiles_g + tile) * kTileTop + lane;
      a.tile_top[ti] = best;
      a.tile_top_id[ti] = best_id;
    }
  }
}

// Packed row piece: 8 elements of one row (16 B of bf16 or 32 B of fp32).
template <typename T> struct Piece;
template <> struct Piece<uint16_t> {
  u32x4_t v;
  __device__ void load(const uint16_t* p) { v = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ void load_nt(const uint16_t* p) { v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)); }
  __device__ void zero() { v = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ void unpack(float (&o)[8]) const {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};
template <> struct Piece<float> {
  u32x4_t v0, v1;
  __device__ void load(const float* p) {
    v0 = *reinterpret_cast<const u32x4_t*>(p);
    v1 = *reinterpret_cast<const u32x4_t*>(p + 4);
  }
  __device__ void load_nt(const float* p) {
    v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + 4));
  }
  __device__ void zero() { v0 = u32x4_t{0u, 0u, 0u, 0u}; v1 = v0; }
  __device__ void unpack(float (&o)[8]) const {
    o[0] = __uint_as_float(v0.x); o[1] = __uint_as_float(v0.y); o[2] = __uint_as_float(v0.z); o[3] = __uint_as_float(v0.w);
    o[4] = __uint_as_float(v1.x); o[5] = __uint_as_float(v1.y); o[6] = __uint_as_float(v1.z); o[7] = __uint_as_float(v1.w);
  }
};

// ============================================================================ estimation
// The first workgroups of the select launch, ahead of the B*Hq select workgroups: estimation
// workgroup x takes the score tiles [e T / E, (e + 1) T / E) of KV group bg (x = bg E + e; T tiles of 128 clusters,
// E = est_blocks_g workgroups per group) and folds, for every query head h of the group,
// m = max over the non-empty clusters of l_c = scale <q_h, mu_c>, den = sum n_c exp(l_c - m) and
// num = sum exp(l_c - m) SV_c (n_c exp(l_c) SV_c / n_c per cluster).  The scores are the score
// kernel's fp32 scores (decoded from their order keys) and m comes from its per-tile maxima.
// These workgroups need no selection, so they stream the value sums while the select
// workgroups, one per query head, leave most CUs idle; each keeps two passes of rows in flight
// and writes one partial per head.
// Buffer resource of a byte range (gfx9 descriptor: raw buffer, no stride, dword 3 0x00020000):
// loads address it with 32-bit offsets from a scalar base, and reads past its end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kStreamNT = 2;        // buffer-load cache policy: non-temporal (streamed once)

// Eight elements of one value-sum row (16 B of bf16, two 16 B pieces of fp32), as raw bits,
// read through a buffer resource with a 32-bit offset.
template <typename T> struct Oct;
template <> struct Oct<uint16_t> {
  u32x4_t v;
  __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t vo, int so) {
    v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, kStreamNT));
  }
  __device__ void unpack(float (&o)[8]) const {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};
template <> struct Oct<float> {
  u32x4_t v0, v1;
  __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t vo, int so) {
    v0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, kStreamNT));
    v1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, vo + 16u, so, kStreamNT));
  }
  __device__ void unpack(float (&o)[8]) const {
    o[0] = __uint_as_float(v0.x); o[1] = __uint_as_float(v0.y); o[2] = __uint_as_float(v0.z); o[3] = __uint_as_float(v0.w);
    o[4] = __uint_as_float(v1.x); o[5] = __uint_as_float(v1.y); o[6] = __uint_as_float(v1.z); o[7] = __uint_as_float(v1.w);
  }
};

// Passes of value-sum rows in flight per estimation wave.  Deeper rings (6, 8) measured slower:
// the extra requests in flight lengthen the memory round trips of the select workgroups that
// share the launch more than they speed up the stream.  1024-thread workgroups (more than 16384
// clusters per KV head) keep two passes in flight: twice the rows per pass, and at 1M tokens
// the launch took 29.7 us with four passes, 28.6 with three and 27.5 with two.
constexpr int kEstRing = 4;
template <int NT> constexpr int est_ring() { return NT >= 1024 ? 2 : kEstRing; }

// f(integral_constant<int, I>) for I = B .. E - 1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <typename T, int NT>
__device__ void est_block(const DecodeArgs& a, int x, float* part /* [NT / 64][2][kD] */,
                          float* sh /* >= 4 + 4 (NT / 64) floats */) {
  // lane (lr = lane & 15, lg = lane >> 4) of wave wv holds dims [8 lr, 8 lr + 8) of row
  // p0 + 4 wv + lg of each pass, NBUF passes in flight (16 KB each per 1024-thread workgroup in bf16)
  // (the select kernel runs one such workgroup per CU, or two of 512 threads)
  constexpr int NW = NT / 64, PASS = NW * 4, NBUF = est_ring<NT>();
  constexpr uint32_t kRow = kD * sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int E = a.est_blocks_g, tiles = a.tiles_g;
  const int bg = x / E, e = x - bg * E;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv, G = a.G, C = a.C;
  const int t0 = (int)((int64_t)e * tiles / E), t1 = (int)((int64_t)(e + 1) * tiles / E);
  const int c0 = t0 * kScoreTile, n = min(C, t1 * kScoreTile) - c0;      // n >= 1 (E <= tiles)
  // the range's value sums, the group's score keys and the range's sizes, as buffer resources:
  // rows past the range read 0 (value sums, sizes) or other clusters' keys, all weighted 0
  const __amdgpu_buffer_rsrc_t r_sv = byte_range(static_cast<const T*>(a.sv) + ((size_t)bg * C + c0) * kD, (uint32_t)n * kRow);
  const __amdgpu_buffer_rsrc_t r_key = byte_range(a.keys + ((size_t)b * a.Hq + (size_t)g * G) * C, (uint32_t)(G * C) * 4u);
  const __amdgpu_buffer_rsrc_t r_sz = byte_range(a.sizes + (size_t)bg * C + c0, (uint32_t)n * 4u);
  const size_t slot = (size_t)bg * E + e;
  for (int h0 = 0; h0 < G; h0 += 4) {
    // Lane lr < 4 of a row group also weighs the row for head h0 + lr (the other lanes copy its
    // weight), so that a lane holds one score key per row.
    const int hl = lr & 3;
    const bool head_live = h0 + hl < G;
    const uint32_t vo_sv = (uint32_t)(4 * wv + lg) * kRow + 8u * sizeof(T) * lr;
    const uint32_t vo_key = ((uint32_t)min(h0 + hl, G - 1) * (uint32_t)C + (uint32_t)c0 + (uint32_t)(4 * wv + lg)) * 4u;
    const uint32_t vo_sz = (uint32_t)(4 * wv + lg) * 4u;
    Oct<T> vr[NBUF];
    uint32_t kk[NBUF];
    float nn[NBUF];
    auto issue = [&](auto buf, int p0) {
      vr[buf].load(r_sv, vo_sv, p0 * (int)kRow);
      kk[buf] = __builtin_amdgcn_raw_buffer_load_b32(r_key, vo_key, p0 * 4, 0);
      nn[buf] = (float)(int)__builtin_amdgcn_raw_buffer_load_b32(r_sz, vo_sz, p0 * 4, 0);
    };
    // m of each head of the chunk: the largest of its tiles' best scores (key 0: no cluster).
    // The first tile maxima are requested before the ring's first passes, which need no m and
    // are in flight while m is formed.
    const uint32_t* tt = a.tile_top + ((size_t)b * a.Hq + (size_t)g * G + h0 + (wv & 3)) * tiles * kTileTop;
    const bool m_lane = wv < 4 && h0 + wv < G;
    const uint32_t k_first = (m_lane && t0 + lane < t1) ? tt[(size_t)(t0 + lane) * kTileTop] : 0u;
    static_for<0, NBUF - 1>([&](auto i) { issue(i, i * PASS); });
    if (wv < 4) {
      float mx = (k_first != 0u) ? f32_from_order_key(k_first) * a.scale : -INFINITY;
      if (m_lane) {
        for (int t = t0 + lane + 64; t < t1; t += 64) {
          const uint32_t k = tt[(size_t)t * kTileTop];
          if (k != 0u) mx = fmaxf(mx, f32_from_order_key(k) * a.scale);
        }
      }
      mx = wave_max(mx);
      if (lane == 0) sh[wv] = mx;
    }
    __syncthreads();
    const float m_own = sh[hl];
    float acc[4][8], den = 0.f;
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
    auto consume = [&](auto buf, int p0) {
      const bool live = p0 + 4 * wv + lg < n;
      const uint32_t k = kk[buf];
      // exp(-inf) = 0 for rows past the range, empty clusters and heads past the group (no branch)
      const float w_own = __expf((live && k != 0u && head_live) ? f32_from_order_key(k) * a.scale - m_own : -INFINITY);
      if (lr < 4) den += w_own * nn[buf];
      float v[8];
      vr[buf].unpack(v);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float wt = __shfl(w_own, (lane & 48) + h);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] += wt * v[j];
      }
      __builtin_amdgcn_sched_barrier(0);     // keep each pass's weights from being hoisted into the last
    };
    // a ring of NBUF passes (the first NBUF - 1 issued above): the loads of pass p + NBUF - 1 are
    // issued before pass p is folded; passes past the range read zeros (no memory access) and
    // are weighted 0
    for (int p0 = 0; p0 < n; p0 += NBUF * PASS) {
      static_for<0, NBUF>([&](auto i) {
        constexpr int I = decltype(i)::value;
        issue(std::integral_constant<int, (I + NBUF - 1) % NBUF>{}, p0 + (I + NBUF - 1) * PASS);
        consume(i, p0 + i * PASS);
      });
    }
    // den of head h0 + h: the lanes lr = h of the row groups; the numerators over the four row
    // groups of a wave (lane shuffles), then over the waves through LDS, two heads a round
    float dh[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) dh[h] = wave_sum(lr == h ? den : 0.f);
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[h][j] += __shfl_xor(acc[h][j], 16);
        acc[h][j] += __shfl_xor(acc[h][j], 32);
      }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < 4; ++h) sh[4 + 4 * wv + h] = dh[h];
    }
#pragma unroll
    for (int hh = 0; hh < 4; hh += 2) {
      if (lg == 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) part[(wv * 2 + u) * kD + 8 * lr + j] = acc[hh + u][j];
      }
      __syncthreads();
      if (tid < 2 * kD) {
        const int u = tid / kD, d = tid - u * kD, h = h0 + hh + u;
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) sum += part[(ww * 2 + u) * kD + d];
        if (h < G) a.est_num[(slot * G + h) * kD + d] = sum;
      }
      if (hh == 0 && tid < 4 && h0 + tid < G) {
        float dn = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) dn += sh[4 + 4 * ww + tid];
        a.est_md[(slot * G + h0 + tid) * 2] = sh[tid];
        a.est_md[(slot * G + h0 + tid) * 2 + 1] = dn;
      }
      __syncthreads();
    }
  }
}

// ============================================================================ k_select
// Block size of the select: 512 threads beyond 256 heads (two heads per CU then run at once) or
// when two blocks fit one CU's LDS (select_half_blocks), otherwise 1024.
constexpr int kSelThreadsFew = 1024, kSelThreadsMany = 512;
constexpr int kSmallBand = 64;      // bands up to one wave are resolved by direct ranking
constexpr int kSumCap = 4096;       // tile summaries (8 per 128-cluster tile) staged in LDS
constexpr int kCandCap = 2048;      // candidate clusters ranked in LDS
constexpr int kFullCap = 256;       // tiles scanned in full
constexpr int kBins = 2048;         // histogram bins over [min, max] of the ranked scores
constexpr int kPubPT = 1;           // retrieved clusters per thread in one publishing round (lanes
                                    // take consecutive entries, so the list stores coalesce)

// Radix bin of the k-th largest key: each thread owns 256 / NT consecutive bins in
// descending order, so an exclusive scan over the threads gives the count above each thread's
// bins; the one bin with excl < rem <= incl is chosen.
template <int NT>
__device__ __forceinline__ void radix_pick(const uint32_t* hist, int rem, int* scr, int* out_bin,
                                           int* out_above) {
  const int tid = threadIdx.x;
  constexpr int per = (256 + NT - 1) / NT;
  int v = 0;
  for (int j = 0; j < per; ++j) { const int bin = 255 - per * tid - j; if (bin >= 0) v += (int)hist[bin]; }
  int tot;
  int run = block_exclusive_scan<NT>(v, scr, &tot);
  if (run < rem && rem <= run + v) {
    for (int j = 0; j < per; ++j) {
      const int bin = 255 - per * tid - j;
      const int hb = (int)hist[bin];
      if (run + hb >= rem) { scr[20] = bin; scr[21] = run; break; }
      run += hb;
    }
  }
  __syncthreads();
  *out_bin = scr[20];
  *out_above = scr[21];
  __syncthreads();
}

// Threshold key of the k-th largest of n keys (1 <= k <= n): afterwards exactly k - *rem_out keys
// are strictly greater than the returned key and at least *rem_out keys equal it.
template <int NT, typename K, typename Get>
__device__ K block_radix_select(int n, int k, Get get, uint32_t* hist, int* scr, int* rem_out) {
  K prefix = 0, mask = 0;
  int rem = k;
  for (int shift = (int)sizeof(K) * 8 - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const K key = get(i);
      if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    int bin, above;
    radix_pick<NT>(hist, rem, scr, &bin, &above);
    prefix |= (K)bin << shift;
    rem -= above;
    mask |= (K)255 << shift;
  }
  *rem_out = rem;
  return prefix;
}

// k-th largest (1 <= k <= n) of n score order keys (all non-zero): a kBins histogram over
// [min, max] of the scores gives the bin of the k-th largest, whose keys are then ranked by one
// wave (a radix select over the keys covers a bin of more than 64).  `bl` holds >= 64 keys.
// Histogram stage shared by the threshold searches below: over the non-zero ones of n score
// order keys (0 marks an empty cluster and is skipped), kBins bins over [min, max] of their
// scores; returns the bin holding the k-th largest (1 <= k <= #non-zero) and how many keys lie in
// higher bins.
struct KthBin { int bin, above; float mn, inv; };   // bin -1: fewer than k non-zero keys
template <int NT, typename Get>
__device__ KthBin kth_bin(int n, int k, Get get, uint32_t* hist, int* iscr, float* fred, int* sh_i) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float mx = -INFINITY, mn = INFINITY;
  for (int i = tid; i < n; i += NT) {
    const uint32_t key = get(i);
    if (key == 0u) continue;
    const float s = f32_from_order_key(key);
    mx = fmaxf(mx, s);
    mn = fminf(mn, s);
  }
  mx = wave_max(mx);
  mn = -wave_max(-mn);
  for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
  if (lane == 0) { fred[2 * wv] = mx; fred[2 * wv + 1] = mn; }
  if (tid == 0) sh_i[4] = 0;                       // key counter of kth_largest_key's small bin
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) { mx = fmaxf(mx, fred[2 * i]); mn = fminf(mn, fred[2 * i + 1]); }
  KthBin r;
  r.mn = mn;
  r.inv = mx > mn ? (float)(kBins - 1) / (mx - mn) : 0.f;
  for (int i = tid; i < n; i += NT) {
    const uint32_t key = get(i);
    if (key == 0u) continue;
    const float s = f32_from_order_key(key);
    atomicAdd(&hist[min(kBins - 1, max(0, (int)((s - r.mn) * r.inv)))], 1u);
  }
  __syncthreads();
  // threshold bin: thread t owns bins kBins-1-BPT*t .. (descending)
  constexpr int BPT = (kBins + NT - 1) / NT;
  int v = 0;
  for (int j = 0; j < BPT; ++j) { const int bin = kBins - 1 - BPT * tid - j; if (bin >= 0) v += (int)hist[bin]; }
  int tot;
  int run = block_exclusive_scan<NT>(v, iscr, &tot);
  if (run < k && k <= run + v) {
    for (int j = 0; j < BPT; ++j) {
      const int bin = kBins - 1 - BPT * tid - j;
      const int hb = (int)hist[bin];
      if (run + hb >= k) { sh_i[0] = bin; sh_i[1] = run; break; }
      run += hb;
    }
  }
  __syncthreads();
  r.bin = tot >= k ? sh_i[0] : -1;
  r.above = sh_i[1];
  return r;
}

__device__ __forceinline__ int bin_of(const KthBin& kb, uint32_t key) {
  return min(kBins - 1, max(0, (int)((f32_from_order_key(key) - kb.mn) * kb.inv)));
}

// k-th largest (k >= 1) of the non-zero ones of n score order keys, 0 when fewer than k are
// non-zero: the histogram bin of the k-th largest, whose keys are then ranked by one wave (a radix
// select over the keys covers a bin of more than 64).  `bl` holds >= 64 keys.
template <int NT, typename Get>
__device__ uint32_t kth_largest_key(int n, int k, Get get, uint32_t* hist, uint32_t* bl, int* iscr,
                                    float* fred, int* sh_i) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const KthBin kb = kth_bin<NT>(n, k, get, hist, iscr, fred, sh_i);
  if (kb.bin < 0) return 0u;
  const int rem = k - kb.above;
  const int nb = (int)hist[kb.bin];
  if (nb <= 64) {
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = get(i);
      if (key != 0u && bin_of(kb, key) == kb.bin) bl[atomicAdd(&sh_i[4], 1)] = key;
    }
    __syncthreads();
    if (wv == 0) {
      const uint32_t key = lane < nb ? bl[lane] : 0u;
      int gt = 0, ge = 0;
      for (int j = 0; j < nb; ++j) { const uint32_t kj = bl[j]; gt += kj > key; ge += kj >= key; }
      if (lane < nb && gt < rem && rem <= ge) sh_i[3] = (int)key;
    }
    __syncthreads();
    return (uint32_t)sh_i[3];
  }
  int rr;
  return block_radix_select<NT, uint32_t>(n, k, get, hist, iscr, &rr);
}

// For one wave (no block barriers): the k-th largest (k >= 1) of n <= 64 KR order keys get(i),
// given that at least k of them are >= L > 0.  Returns L when fewer than k keys exceed L.
// Otherwise the k-th largest is the e-th smallest key above L, e = #(keys > L) - k + 1: for e <= 8
// by walking up the distinct keys above L (a wave minimum and a tie count each), else a 256-bin
// histogram over (L, max] names its bin and the bin's keys are ranked directly.  The keys are
// read once, KR per lane, and kept in registers.  Returns 0 when n > 64 KR or when that
// bin holds more than 64 keys (the caller then searches with the whole block).  `hist` holds
// >= 256 counters and `bl` >= 64 keys of LDS that no other wave touches meanwhile.
template <int KR, typename Get>
__device__ uint32_t wave_kth_above(int n, int k, uint32_t L, Get get, uint32_t* hist, uint32_t* bl) {
  constexpr int NB = 256;
  if (n > 64 * KR) return 0u;
  const int lane = threadIdx.x & 63;
  uint32_t kr[KR];
#pragma unroll
  for (int r = 0; r < KR; ++r) { const int i = lane + 64 * r; kr[r] = i < n ? get(i) : 0u; }
#pragma unroll
  for (int j = 0; j < NB / 64; ++j) hist[lane + 64 * j] = 0u;
  int d = 0;
  uint32_t mk = 0u;
#pragma unroll
  for (int r = 0; r < KR; ++r) if (kr[r] > L) { ++d; mk = max(mk, kr[r]); }
  d = wave_isum(d);
  if (d < k) return L;
  mk = wave_umax(mk);
  const int e = d - k + 1;
  if (e <= 8) {
    // few keys to pass over: walk up the distinct keys above L, smallest first, counting ties
    uint32_t v = L;
    int left = e;
    for (int it = 0; it < 8; ++it) {
      uint32_t mn = 0xffffffffu;
#pragma unroll
      for (int r = 0; r < KR; ++r) if (kr[r] > v) mn = min(mn, kr[r]);
      mn = ~wave_umax(~mn);
      int c = 0;
#pragma unroll
      for (int r = 0; r < KR; ++r) c += kr[r] == mn ? 1 : 0;
      c = wave_isum(c);
      if (c >= left) return mn;
      left -= c;
      v = mn;
    }
  }
  const float lo = f32_from_order_key(L), hi = f32_from_order_key(mk);
  const float inv = hi > lo ? (float)NB / (hi - lo) : 0.f;
  auto bin_of_key = [&](uint32_t key) { return min(NB - 1, max(0, (int)((f32_from_order_key(key) - lo) * inv))); };
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < KR; ++r) if (kr[r] > L) atomicAdd(&hist[bin_of_key(kr[r])], 1u);
  wave_lds_sync();
  // lane j holds bins 4 j .. 4 j + 3, ascending; the bin holding the e-th smallest
  const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
  const int v = (int)(h0 + h1 + h2 + h3);
  const int inc = wave_inclusive_scan(v), exc = inc - v;
  const uint64_t own = __ballot(exc < e && e <= inc);
  const int owner = __ffsll((unsigned long long)own) - 1;
  int bin = 0, below = exc, nb = (int)h0;
  if (below + (int)h0 < e) { below += (int)h0; bin = 1; nb = (int)h1;
    if (below + (int)h1 < e) { below += (int)h1; bin = 2; nb = (int)h2;
      if (below + (int)h2 < e) { below += (int)h2; bin = 3; nb = (int)h3; } } }
  bin = __builtin_amdgcn_readlane(4 * lane + bin, owner);
  below = __builtin_amdgcn_readlane(below, owner);
  nb = __builtin_amdgcn_readlane(nb, owner);
  if (nb > 64) return 0u;
  int run = 0;
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    const bool take = kr[r] > L && bin_of_key(kr[r]) == bin;
    const uint64_t m = __ballot(take);
    if (take) bl[run + __popcll(m & ((1ull << lane) - 1ull))] = kr[r];
    run += __popcll(m);
  }
  wave_lds_sync();
  // the rem-th smallest key of the bin
  const int rem = e - below;
  const uint32_t key = lane < nb ? bl[lane] : 0u;
  int lt = 0, le = 0;
  for (int j = 0; j < nb; ++j) { const uint32_t kj = bl[j]; lt += kj < key; le += kj <= key; }
  const uint64_t hit = __ballot(lane < nb && lt < rem && rem <= le);
  return (uint32_t)__builtin_amdgcn_readlane((int)key, __ffsll((unsigned long long)hit) - 1);
}

// ---- ranking and fp64 reductions of the accuracy-bounded select
// A key of the canonical order of the bounded zone: (-sigma, id) as (order key of sigma, id).
struct CanonKey {
  uint64_t k;
  int id;
};
__device__ __forceinline__ bool canon_gt(const CanonKey& x, const CanonKey& y) {
  return x.k > y.k || (x.k == y.k && x.id < y.id);
}
__device__ __forceinline__ uint64_t bcast_lane(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ CanonKey bcast_lane(const CanonKey& v, int l) {
  return {bcast_lane(v.k, l), __builtin_amdgcn_readlane(v.id, l)};
}

// Ranks in descending order (under gt, a strict total order; the keys are distinct) of n <=
// EPT * NT keys, thread t holding keys e * NT + t.  Every run of 64 consecutive keys belongs to
// one wave: its keys are ranked among themselves and stored in that order through put(position,
// key); a key's rank is its rank in its run plus, for every other run, the number of keys above
// it, found by a binary search through get(position).  O(n log 64) LDS reads per key against
// O(n) for direct counting.  Within a run the keys are compared either from lane broadcasts or,
// when orig(i) reads key i from LDS (kOrig), from broadcast LDS reads, which pipeline; the sorted
// runs may then overwrite those keys (a barrier separates the two).
template <int NT, int EPT, bool kOrig, typename K, typename Gt, typename Put, typename Get, typename Orig>
__device__ __forceinline__ void block_rank_desc(int n, const K (&key)[EPT], int (&rank)[EPT], Gt gt,
                                                Put put, Get get, Orig orig) {
  const int tid = threadIdx.x, lane = tid & 63;
  int rr[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = e * NT + tid, base = i - lane;
    int r = 0;
    if (base < n) {                                  // uniform over the wave
      const int len = min(64, n - base);
      if constexpr (kOrig) {
#pragma unroll 8
        for (int l = 0; l < len; ++l) r += gt(orig(base + l), key[e]) ? 1 : 0;
      } else {
        for (int l = 0; l < len; ++l) r += gt(bcast_lane(key[e], l), key[e]) ? 1 : 0;
      }
    }
    rr[e] = r;
  }
  if constexpr (kOrig) __syncthreads();
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = e * NT + tid;
    if (i < n) put((i - lane) + rr[e], key[e]);
  }
  __syncthreads();
  const int runs = (n + 63) / 64;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = e * NT + tid;
    rank[e] = 0;
    if (i >= n) continue;
    const int own = i >> 6;
    int tot = rr[e];
    for (int r = 0; r < runs; ++r) {
      if (r == own) continue;
      const int len = min(64, n - 64 * r);
      int pos = 0;                                   // keys [0, pos) of run r are above key[e]
#pragma unroll
      for (int st = 32; st >= 1; st >>= 1) {
        const int q = pos + st - 1;
        if (q < len && gt(get(64 * r + q), key[e])) pos += st;
      }
      if (pos < len && gt(get(64 * r + pos), key[e])) ++pos;
      tot += pos;
    }
    rank[e] = tot;
  }
  __syncthreads();
}

// NS sums and one maximum over the block with a single pair of barriers; scratch holds
// (NS + 1) * NT / 64 floats.
template <int NT, int NS>
__device__ __forceinline__ void block_sums_max(float (&v)[NS], float& mx, float* scratch) {
  constexpr int nw = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NS; ++i) v[i] = wave_sum(v[i]);
  mx = wave_max(mx);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) scratch[i * nw + w] = v[i];
    scratch[NS * nw + w] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < nw; ++j) r += scratch[i * nw + j];
    v[i] = r;
  }
  float m = scratch[NS * nw];
#pragma unroll
  for (int j = 1; j < nw; ++j) m = fmaxf(m, scratch[NS * nw + j]);
  mx = m;
  __syncthreads();
}

// Block-wide exclusive prefix sum of any arithmetic type (lane shifts, then the wave totals in
// LDS scratch of NT / 64 entries); *total receives the block sum.
template <int NT, typename V>
__device__ __forceinline__ V block_exclusive_scan_any(V v, V* scratch, V* total) {
  constexpr int nw = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  V inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const V o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  V before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < nw; ++i) {
    const V t = scratch[i];
    before += i < w ? t : V(0);
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return before + inc - v;
}
template <int NT>
__device__ __forceinline__ double block_sum_d(double v, double* scratch) {
  double tot;
  block_exclusive_scan_any<NT, double>(v, scratch, &tot);
  return tot;
}
template <int NT>
__device__ __forceinline__ double block_max_d(double v, double* scratch) {
  constexpr int nw = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmax(v, __shfl_xor(v, m));
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < nw; ++i) r = fmax(r, scratch[i]);
  __syncthreads();
  return r;
}

// Canonical fp64 score of the query (fp64 copy in LDS) and one centroid row: exact products
// summed in ascending coordinate order, no contraction.  The row is fetched in four batches.
template <typename T>
__device__ __forceinline__ double canonical_score_row(const double* qd, const T* row) {
#pragma clang fp contract(off)
  double acc = 0.0;
#pragma unroll 1
  for (int j0 = 0; j0 < kD; j0 += 32) {
    float x[32];
#pragma unroll
    for (int u = 0; u < 32; u += 8) {
      float t[8];
      St<T>::load8(row + j0 + u, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[u + e] = t[e];
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const double p = qd[j0 + e] * (double)x[e];
      acc = acc + p;
    }
  }
  return acc;
}

// Visits the coordinates of one centroid row in ascending order, f(j, value), with the row's
// loads issued in batches of kPieces raw 16-byte pieces, kept packed until used: one memory round
// trip per batch and 4 kPieces registers of row data.
template <typename T, int kPieces, typename F>
__device__ __forceinline__ void row_visit(const T* row, F&& f) {
  constexpr int kPer = 16 / (int)sizeof(T);             // elements per piece
  constexpr int kBatch = kPieces * kPer;                // elements per batch
#pragma unroll
  for (int j0 = 0; j0 < kD; j0 += kBatch) {
    u32x4_t r[kPieces];
#pragma unroll
    for (int i = 0; i < kPieces; ++i) r[i] = *reinterpret_cast<const u32x4_t*>(row + j0 + i * kPer);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2) {
          f(j0 + i * 8 + 2 * e, __uint_as_float(w[e] << 16));
          f(j0 + i * 8 + 2 * e + 1, __uint_as_float(w[e] & 0xffff0000u));
        } else {
          f(j0 + i * 4 + e, __uint_as_float(w[e]));
        }
      }
    }
  }
}

// <q, row> in fp64 with four partial sums: not the canonical rounding, but within d 2^-53
// sum |q_j row_j| of it (about 1e-13 of the score here), which moves a cluster's weight by a
// relative 1e-13 -- for sums of terms, where the value matters and not the rounding.
template <typename T>
__device__ __forceinline__ double score_row_f64(const double* qd, const T* row) {
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  row_visit<T, 16>(row, [&](int j, float x) { acc[j & 3] = fma(qd[j], (double)x, acc[j & 3]); });
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// canonical_score_row with the row loaded by row_visit (same products, same order of additions).
template <typename T>
__device__ __forceinline__ double canonical_score_row_unrolled(const double* qd, const T* row) {
  double acc = 0.0;
  row_visit<T, 8>(row, [&](int j, float x) {
#pragma clang fp contract(off)
    acc = acc + qd[j] * (double)x;
  });
  return acc;
}

// Pointers into LDS (address space 3) and global memory (1) for the parameters of an out-of-line
// function: through plain pointers its accesses would be flat ones, which wait for every memory
// operation in flight.
template <typename X> using lds_ptr = __attribute__((address_space(3))) X*;
template <typename X> using gbl_ptr = __attribute__((address_space(1))) X*;

// The zone size of the accuracy-bounded select decided in fp64, when the fp32 decision could not
// be certified: every non-empty cluster's err and lo in fp64, term by term as the bound defines
// them (the list's clusters from their canonical scores, the others' from score_row_f64); the
// selected list (the canonical top k_eff, ids zi[0 .. k_eff)) ranked by (-sigma, id); and the
// smallest j with A(j) = (err summed after the first j) / (sum of every lo) <= eps, the cap k_eff
// when none.  Leaves the first j of the canonical order in `bits` (which holds the list on entry)
// and returns j.  zo (k_eff 8-byte slots) and run_ids (k_eff ints) are LDS scratch; every thread
// of the block calls it.  Out of line, so that its registers do not weigh on the select.
template <typename T, int NT>
__device__ __attribute__((noinline)) int bounded_zone_fp64(
    gbl_ptr<const uint32_t> keys_g, gbl_ptr<const T> mu_g, gbl_ptr<const int32_t> szg_g, gbl_ptr<const float> rdg_g,
    gbl_ptr<const float> vng_g, double vall, double sc, double uu, double eps, int C, int W32, int k_eff,
    lds_ptr<const double> qd_l, lds_ptr<const int> zi_l, lds_ptr<uint64_t> zo_l, lds_ptr<int> run_ids_l,
    lds_ptr<uint32_t> bits_l, lds_ptr<double> dscr_l, lds_ptr<float> fred_l) {
#pragma clang fp contract(off)
  const uint32_t* keys = (const uint32_t*)keys_g;
  const T* mu = (const T*)mu_g;
  const int32_t* szg = (const int32_t*)szg_g;
  const float* rdg = (const float*)rdg_g;
  const float* vng = (const float*)vng_g;
  const double* qd = (const double*)qd_l;
  const int* zi = (const int*)zi_l;
  uint64_t* zo = (uint64_t*)zo_l;
  int* run_ids = (int*)run_ids_l;
  uint32_t* bits = (uint32_t*)bits_l;
  double* dscr = (double*)dscr_l;
  float* fred = (float*)fred_l;
  constexpr int EPT = kBoundedMaxTopK / NT;
  const int tid = threadIdx.x;
  double qn2 = 0.0;
#pragma unroll 8
  for (int j = 0; j < kD; ++j) qn2 = qn2 + qd[j] * qd[j];
  const double qn = sqrt(qn2);
  double s64[EPT];
  CanonKey ck[EPT];
  double smax = -INFINITY;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int p = e * NT + tid;
    s64[e] = 0.0;
    ck[e] = CanonKey{0ull, 0x7fffffff};
    if (p < k_eff) {
      s64[e] = canonical_score_row_unrolled<T>(qd + opaque_zero(), mu + (size_t)zi[p] * kD);
      ck[e] = CanonKey{f64_order_key(s64[e]), zi[p]};
      smax = fmax(smax, s64[e]);
    }
  }
  const double mstar = sc * block_max_d<NT>(smax, dscr);
  auto terms64 = [&](double s, double n, double r, double vc, double& err, double& lo) {
#pragma clang fp contract(off)
    const double x = sc * qn * r;
    const double w = n * exp(sc * s - mstar);
    const double av = w * expm1(x);
    err = av * (vc + (1.0 + uu) * vall) + w * uu * vc;
    lo = w * exp(-x);
  };
  // the clusters outside the list; each cluster's key, size, radius and value norm are fetched
  // one iteration ahead, so that a live cluster costs the one round trip of its row
  double tout = 0.0, dsum = 0.0;
  uint32_t kn = 0u;
  float nn = 0.f, rn = 0.f, vn = 0.f;
  if (tid < C) { kn = keys[tid]; nn = (float)szg[tid]; rn = rdg[tid]; vn = vng[tid]; }
  for (int c = tid; c < C; c += NT) {
    const uint32_t kc = kn;
    const float nc = nn, rc = rn, vc = vn;
    if (c + NT < C) { kn = keys[c + NT]; nn = (float)szg[c + NT]; rn = rdg[c + NT]; vn = vng[c + NT]; }
    if (kc == 0u || ((bits[c >> 5] >> (c & 31)) & 1u)) continue;
    double e1, l1;
    terms64(score_row_f64<T>(qd + opaque_zero(), mu + (size_t)c * kD), (double)nc, (double)rc, (double)vc, e1, l1);
    tout = tout + e1;
    dsum = dsum + l1;
  }
  double el[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    el[e] = 0.0;
    if (e * NT + tid < k_eff) {
      const int c = ck[e].id;
      double l1;
      terms64(s64[e], (double)szg[c], (double)rdg[c], (double)vng[c], el[e], l1);
      dsum = dsum + l1;
    }
  }
  const double t_out = block_sum_d<NT>(tout, dscr);
  const double d_all = block_sum_d<NT>(dsum, dscr);
  int rk[EPT];
  block_rank_desc<NT, EPT, false>(k_eff, ck, rk, [](const CanonKey& x, const CanonKey& y) { return canon_gt(x, y); },
                                  [&](int p, const CanonKey& k) { zo[p] = k.k; run_ids[p] = k.id; },
                                  [&](int p) { return CanonKey{zo[p], run_ids[p]}; }, [](int) { return CanonKey{}; });
  double* ez = reinterpret_cast<double*>(zo);           // err in canonical order
#pragma unroll
  for (int e = 0; e < EPT; ++e) if (e * NT + tid < k_eff) ez[rk[e]] = el[e];
  __syncthreads();
  // T(j) = t_out + the err of canonical positions j .. k_eff - 1 (thread t: positions
  // k_eff - 1 - (t EPT + e)), then A(j) = T(j) / d_all
  double dl[EPT], drun = 0.0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int p = k_eff - 1 - (tid * EPT + e);
    drun = drun + (p >= 0 ? ez[p] : 0.0);
    dl[e] = drun;
  }
  double dtot;
  const double dbefore = block_exclusive_scan_any<NT, double>(drun, dscr, &dtot);
  int kb = k_eff;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int p = k_eff - 1 - (tid * EPT + e);
    if (p >= 0 && (t_out + (dbefore + dl[e])) / d_all <= eps) kb = min(kb, p);
  }
  const int kz = (int)-block_max<NT>(-(float)kb, fred);
  if (kz < k_eff) {
    for (int w = tid; w < W32; w += NT) bits[w] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (e * NT + tid < k_eff && rk[e] < kz) { const int c = ck[e].id; atomicOr(&bits[c >> 5], 1u << (c & 31)); }
    __syncthreads();
  }
  return kz;
}

// Per query head: the retrieval zone is the k_eff = min(top_k, #non-empty) non-empty clusters
// first in the order (-sigma_c, c).  With t the k_eff-th largest fp32 score and delta a bound on
// |fp32 score - canonical fp64 score|, clusters above t + 2 delta are in, those below t - 2 delta
// are out, and the band in between is re-scored canonically and ranked by (-sigma, id).
//
// One pass over the head's scores: the score kernel kept the 8 best scores of every 128-cluster
// tile, and the k_eff-th largest of those is a lower bound L <= t; the pass collects every
// cluster scoring >= L - 2 delta (t, the band and everything above it) into LDS, and t, the
// in/band split and the band ranking then run on that short list.  If the list overflows (ties
// or a head whose best clusters crowd a few tiles) t is found by a radix select over all scores
// and the split by a second pass.  The head's list (ascending id: cluster, first row, first
// token, score key) and the entry of every attention workgroup's first token are published last.
static_assert(kMaxGroup * kD <= kCandCap, "a KV group's queries are staged in the candidate arrays");
static_assert(kBoundedMaxTopK <= kCandCap && kBoundedMaxTopK <= kSumCap && kBoundedMaxTopK <= kBins,
              "the bounded select lists its zone in LDS");
// MODE 0: plain decode; 1: the gated, refresh and bounded modes; 2: the bounded mode's second
// launch, for the heads whose zone size the first could not certify in fp32 (it decides them in
// fp64).  Each mode is its own instantiation, so that the plain decode, and the first bounded
// launch, carry no registers of the modes they do not run.
template <typename T, int NT, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void k_select(DecodeArgs a) {
  constexpr bool EXT = MODE != 0, EXACT = MODE == 2;
  extern __shared__ uint32_t dynl[];                 // [W32] retrieved bitmap, [W32] band bitmap
  __shared__ __attribute__((aligned(16))) uint32_t skey[kSumCap];   // tile summaries: score keys
  __shared__ int sid[kSumCap];                       // tile summaries: cluster ids; then the
                                                     // ascending retrieved list
  __shared__ __attribute__((aligned(16))) uint32_t ckey[kCandCap];   // candidates: score keys
  __shared__ __attribute__((aligned(16))) int cidl[kCandCap];        // candidates: cluster ids
  __shared__ __attribute__((aligned(16))) int tfull[kFullCap];   // tiles whose 8 best pass the threshold
  __shared__ __attribute__((aligned(16))) int rl_off[kCandCap];  // retrieved list, by rank: first row, size
  __shared__ __attribute__((aligned(16))) int rl_sz[kCandCap];
  __shared__ uint32_t hist[kBins];
  __shared__ int iscr[48];
  __shared__ float fred[32];
  __shared__ double qd[kD];
  __shared__ int band_lds[kSmallBand];
  __shared__ double gdd[3 * kMaxGroup];              // gated decode: <q, q'>, |q|^2, |q'|^2 per head
  __shared__ double dscr[16];                        // bounded decode: fp64 reduction scratch
  __shared__ int sh_i[8];
  static_assert((NT / 64) * 2 * kD <= kSumCap && 4 + 4 * (NT / 64) <= kSumCap, "estimation scratch");
  if (EXACT && a.bnd_redo[blockIdx.x] == 0) return;   // decided by the first launch
  // the estimation workgroups come first in the grid, so that they start streaming before the
  // select workgroups fill the CUs (batch 16: select launch 60.5 -> 57.4 us)
  const int n_est = (int)gridDim.x - a.B * a.Hq;
  const int bi = (int)blockIdx.x;
  if (!EXACT && bi < n_est) {                        // an estimation workgroup (uniform branch)
    est_block<T, NT>(a, bi, reinterpret_cast<float*>(skey), reinterpret_cast<float*>(sid));
    return;
  }

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bh = EXACT ? bi : bi - n_est;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int g = h / a.G, bg = b * a.Hkv + g;
  // refresh: only the heads whose group attended over its previous zones select again
  if (EXT && a.refresh && a.gate[bg] == 0) return;
  const int C = a.C, W32 = a.W32, tiles = a.tiles_g;
  uint32_t* bits = dynl;
  uint32_t* bbits = dynl + W32;
  const uint32_t* keys = a.keys + (size_t)bh * C;
  const T* qh = static_cast<const T*>(a.q) + (size_t)bh * kD;
  const T* mu = static_cast<const T*>(a.mu) + (size_t)bg * C * kD;
  const int KPT = (C + NT - 1) / NT;          // thread t visits clusters j * NT + t, j < KPT

  // ---- set-up: query, largest centroid norm, non-empty count, tile summaries.  Each thread's
  // first element of each is loaded before any of them is used (indices clamped in range, the
  // value kept only where in range), so that the loads share one round trip; any further
  // elements follow in loops.
  const int nsum = tiles * kTileTop;
  const bool use_sum = nsum <= kSumCap;
  const float* tnorm = a.tile_norm + (size_t)bg * tiles;
  const int* tcnt = a.tile_cnt + (size_t)bg * tiles;
  const uint32_t* ttop = a.tile_top + (size_t)bh * nsum;
  const int* ttid = a.tile_top_id + (size_t)bh * nsum;
  const float q0 = St<T>::f(qh[min(tid, kD - 1)]);
  float tn0 = 0.f;
  int tc0 = 0;
  if (tiles > 0) { tn0 = tnorm[min(tid, tiles - 1)]; tc0 = tcnt[min(tid, tiles - 1)]; }
  uint32_t sk0 = 0u;
  int si0 = 0;
  if (use_sum && nsum > 0) { sk0 = ttop[min(tid, nsum - 1)]; si0 = ttid[min(tid, nsum - 1)]; }
  float qv = 0.f;                             // this thread's part of |q|^2
  if (tid < kD) { qd[tid] = (double)q0; qv = q0 * q0; }
  for (int i = tid + NT; i < kD; i += NT) { const float x = St<T>::f(qh[i]); qd[i] = (double)x; qv += x * x; }
  float mxn = tid < tiles ? tn0 : 0.f;
  int ne = tid < tiles ? tc0 : 0;
  for (int i = tid + NT; i < tiles; i += NT) { mxn = fmaxf(mxn, tnorm[i]); ne += tcnt[i]; }
  if (use_sum) {
    if (tid < nsum) { skey[tid] = sk0; sid[tid] = si0; }
    for (int i = tid + NT; i < nsum; i += NT) { skey[i] = ttop[i]; sid[i] = ttid[i]; }
  }
  // every set-up load has landed: say so to the compiler (vmcnt(0) expcnt(7) lgkmcnt(15)), whose
  // bookkeeping would otherwise keep a conditionally loaded register pending on some paths and,
  // at its next reuse, wait for every later load (the candidates' first rows in flight)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  for (int w = tid; w < 2 * W32; w += NT) dynl[w] = 0u;
  // gated decode: the KV group's current and previous queries, staged (exact in fp32) in the
  // candidate arrays, which are not used before the zone is decided
  float* gq = reinterpret_cast<float*>(ckey);
  float* gp = reinterpret_cast<float*>(cidl);
  if (EXT && a.gated) {
    const size_t row0 = ((size_t)b * a.Hq + (size_t)g * a.G) * kD;
    for (int i = tid; i < a.G * kD; i += NT) {
      gq[i] = St<T>::f(static_cast<const T*>(a.q)[row0 + i]);
      gp[i] = St<T>::f(static_cast<const T*>(a.q_prev)[row0 + i]);
    }
  }
  {
    float v0 = (float)ne, v1 = mxn, v2 = qv;
    v0 = wave_sum(v0); v1 = wave_max(v1); v2 = wave_sum(v2);
    if (lane == 0) { fred[wv] = v0; fred[16 + wv] = v1; hist[wv] = __float_as_uint(v2); }
    __syncthreads();
    float r0 = 0.f, r1 = 0.f, r2 = 0.f;
    for (int i = 0; i < NT / 64; ++i) { r0 += fred[i]; r1 = fmaxf(r1, fred[16 + i]); r2 += __uint_as_float(hist[i]); }
    ne = (int)r0; mxn = r1; qv = sqrtf(r2);
    __syncthreads();
  }
  const int n_ne = ne;
  const int k_eff = min(a.top_k, n_ne);
  // gated decode: the KV group keeps its heads' previous zones when every one of its query heads
  // moved by a cosine of at least tau, <q, q'> / (|q| |q'|) from canonical fp64 sums (ascending
  // coordinate order) with IEEE square roots and division, 0 when either query is zero.  Every
  // head of the group takes the same decision from the same sums.
  bool reuse = false;
  if (EXT && a.gated) {
    if (tid < 3 * a.G) {                      // thread 3 j + {0, 1, 2}: <q_j, q'_j>, |q_j|^2, |q'_j|^2
      const int j = tid / 3, kind = tid - 3 * j;
      const f32x4_t* x = reinterpret_cast<const f32x4_t*>((kind == 2 ? gp : gq) + j * kD);
      const f32x4_t* y = reinterpret_cast<const f32x4_t*>((kind == 1 ? gq : gp) + j * kD);
      // products of fp32 values are exact in fp64, so a fused multiply-add rounds as the sum does
      double acc = 0.0;
#pragma unroll 8
      for (int e = 0; e < kD / 4; ++e) {
        const f32x4_t u = x[e], v = y[e];
        acc = acc + (double)u[0] * (double)v[0];
        acc = acc + (double)u[1] * (double)v[1];
        acc = acc + (double)u[2] * (double)v[2];
        acc = acc + (double)u[3] * (double)v[3];
      }
      gdd[tid] = acc;
    }
    __syncthreads();
    if (tid < 64) {
      bool ok = true;
      if (tid < a.G) {
        const double dq = gdd[3 * tid], n1 = gdd[3 * tid + 1], n2 = gdd[3 * tid + 2];
        const double cs = (n1 == 0.0 || n2 == 0.0) ? 0.0 : dq / (sqrt(n1) * sqrt(n2));
        ok = cs >= (double)a.tau;
      }
      const bool all_ok = __ballot(!ok) == 0ull;
      if (tid == 0) {
        sh_i[6] = all_ok ? 1 : 0;
        if (h == g * a.G) {
          a.gate[bg] = all_ok ? 1 : 0;
          if (a.reused) a.reused[bg] = all_ok ? 1 : 0;
        }
      }
    }
    __syncthreads();
    reuse = sh_i[6] != 0;
  } else if (!(EXT && a.refresh) && tid == 0 && h == g * a.G) {
    a.gate[bg] = 0;                           // a refresh after a plain decode has nothing to do
  }
  int n_reused_ne = 0;              // non-empty clusters of a reused zone

  auto visit_keys = [&](auto&& fn) {           // fn(c, key) for every cluster of this thread
    for (int j0 = 0; j0 < KPT; j0 += 16) {
      uint32_t k[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = (j0 + i) * NT + tid;
        k[i] = c < C ? keys[c] : 0u;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = (j0 + i) * NT + tid;
        if (c < C) fn(c, k[i]);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);         // every load above has landed (as at set-up)
    }
  };

  // delta bounds |fp32 score - canonical fp64 score| for every cluster: fp32 accumulation of d
  // exact-or-rounded products, doubled for an unspecified MFMA summation order
  const double delta = 2.0 * (kD + 2) * 5.9604644775390625e-08 * (double)qv * (1.0 + 1.0 / 1024) *
                           (double)mxn * (1.0 + 1.0 / 1024) + 1e-30;

  // ---- accuracy-bounded zone sizing: error terms of the non-empty clusters in the frame of the
  // largest logit m*: w = n exp(l - m*), a = w (exp(x) - 1) with x = s |q| r_c, lo = w exp(-x),
  // err = a (V_c + (1 + u) V_all) + w u V_c.  A zone Z bounds the error of the output by
  // (sum over the non-empty clusters outside Z of err) / (sum of every lo) before attention.
  float b_mstar = 0.f;
  const float b_vall = EXT && a.bounded ? a.vmax[bg] : 0.f;
  // the terms of cluster c from its score key, size n, radius r and value norm vc
  struct BTerms { float err, lo, ea, eav; };
  auto bound_terms = [&](uint32_t k, float n, float r, float vc) -> BTerms {
    const float x = a.scale * qv * r;
    const float w = n * __expf(f32_from_order_key(k) * a.scale - b_mstar);
    const float ea = w * expm1f(x);
    return {ea * (vc + (1.f + a.u) * b_vall) + w * a.u * vc, w * __expf(-x), ea, ea * vc + w * a.u * vc};
  };
  if (EXT && a.bounded && n_ne > 0) {
    // m*: the largest score, from the tiles' best scores when they are staged
    float m = -INFINITY;
    if (use_sum) {
      for (int t = tid; t < tiles; t += NT) {
        const uint32_t k = skey[t * kTileTop];
        if (k != 0u) m = fmaxf(m, f32_from_order_key(k));
      }
    } else {
      visit_keys([&](int c, uint32_t k) { if (k != 0u) m = fmaxf(m, f32_from_order_key(k)); });
    }
    b_mstar = block_max<NT>(m, fred) * a.scale;
  }

  bool fast_pub = false;            // the retrieved clusters are all LDS candidates
  int co[kCandCap / NT], ce[kCandCap / NT];
  if (reuse) {
    // the previous zone: its ids in [0, C), each once (the bitmap drops repeats)
    const int32_t* sp = a.sel_prev + (size_t)bh * a.top_k;
    int cnt = 0;
    for (int i = tid; i < a.top_k; i += NT) {
      const int c = sp[i];
      if (c >= 0 && c < C) {
        const uint32_t old = atomicOr(&bits[c >> 5], 1u << (c & 31));
        if (!((old >> (c & 31)) & 1u) && keys[c] != 0u) ++cnt;
      }
    }
    n_reused_ne = block_isum<NT>(cnt, iscr);
  } else if (k_eff > 0 && k_eff == n_ne) {
    visit_keys([&](int c, uint32_t k) { if (k != 0u) atomicOr(&bits[c >> 5], 1u << (c & 31)); });
  } else if (k_eff > 0) {
    // ---- L = the k_eff-th largest of the tile summaries: a lower bound of t, and t itself
    // when no tile has its 8th best within 2 delta of L (every score >= L is then a summary)
    float thr_f = -INFINITY;
    uint32_t L = 0u;
    if (use_sum) {
      L = kth_largest_key<NT>(nsum, k_eff, [&](int i) { return skey[i]; }, hist, reinterpret_cast<uint32_t*>(band_lds), iscr, fred, sh_i);
      if (L != 0u) {
        const double thr_d = (double)f32_from_order_key(L) - 2.0 * delta;
        thr_f = (float)thr_d;
        if ((double)thr_f > thr_d) thr_f = nextafterf(thr_f, -INFINITY);
      }
    }
    if (tid == 0) { sh_i[2] = 0; sh_i[5] = 0; sh_i[7] = 0; }
    __syncthreads();
    // ---- candidates: the non-empty clusters scoring >= L - 2 delta (appends wave-aggregated)
    auto append = [&](bool take, uint32_t key, int id) {
      const uint64_t m = __ballot(take);
      if (m == 0ull) return;
      const int leader = __ffsll((unsigned long long)m) - 1;
      int base = 0;
      if (lane == leader) base = atomicAdd(&sh_i[2], __popcll(m));
      base = __builtin_amdgcn_readlane(base, leader);
      if (take) {
        const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
        if (pos < kCandCap) { ckey[pos] = key; cidl[pos] = id; }
      }
    };
    auto passes = [&](uint32_t k) { return k != 0u && f32_from_order_key(k) >= thr_f; };
    bool scan_all = !use_sum;
    if (use_sum) {
      // a tile whose 8th best score is below the threshold has all its candidates among its 8
      // best; the others are scanned in full
      for (int i = tid; i < nsum; i += NT) {
        const int t = i / kTileTop;
        const bool full = passes(skey[t * kTileTop + kTileTop - 1]);
        append(!full && passes(skey[i]), skey[i], sid[i]);
        if (full && i == t * kTileTop) {
          const int q = atomicAdd(&sh_i[5], 1);
          if (q < kFullCap) tfull[q] = t;
        }
      }
      __syncthreads();
      const int n_full = sh_i[5];
      if (n_full > kFullCap) {
        scan_all = true;
        __syncthreads();
        if (tid == 0) sh_i[2] = 0;
        __syncthreads();
      } else {
        for (int j = wv; j < n_full; j += NT / 64) {
          const int t = tfull[j];
          for (int r = lane; r < kScoreTile; r += 64) {
            const int c = t * kScoreTile + r;
            const uint32_t key = c < C ? keys[c] : 0u;
            append(passes(key), key, c);
          }
        }
      }
    }
    if (scan_all) visit_keys([&](int c, uint32_t k) { append(passes(k), k, c); });
    __syncthreads();
    const int n_c = sh_i[2];
    const bool listed = n_c <= kCandCap;
    fast_pub = listed;
    // ---- t = k_eff-th largest score.  The candidates hold every cluster above L and at least
    // k_eff of them score >= L, so t = L when fewer than k_eff candidates score above L; always so
    // when no tile was scanned in full (every cluster above L is then one of the fewer than k_eff
    // summary entries above L).  Otherwise one wave finds t among the candidates above L when
    // there are at most 512 candidates (the block counts them when there are more); the whole
    // block searches the candidates when there are more or that wave's histogram bin is crowded,
    // and every score when the candidates overflowed.
    bool t_is_L = listed && L != 0u && !scan_all && sh_i[5] == 0;
    uint32_t thr = 0u;
    if (listed && L != 0u && !t_is_L && n_c > 64 * 8) {
      int d = 0;
      for (int i = tid; i < n_c; i += NT) d += ckey[i] > L ? 1 : 0;
      t_is_L = block_isum<NT>(d, iscr) < k_eff;
    } else if (listed && L != 0u && !t_is_L) {
      if (wv == 0) {
        const uint32_t r = wave_kth_above<8>(n_c, k_eff, L, [&](int i) { return ckey[i]; }, hist,
                                             reinterpret_cast<uint32_t*>(band_lds));
        if (lane == 0) sh_i[3] = (int)r;
      }
      __syncthreads();
      thr = (uint32_t)sh_i[3];
      t_is_L = thr == L;
    }
    if (t_is_L) {
      thr = L;
    } else if (listed && thr != 0u) {
      // found by the wave
    } else if (listed) {
      thr = kth_largest_key<NT>(n_c, k_eff, [&](int i) { return ckey[i]; }, hist, reinterpret_cast<uint32_t*>(band_lds), iscr, fred, sh_i);
    } else {
      int rr;
      thr = block_radix_select<NT, uint32_t>(C, k_eff, [&](int c) { return keys[c]; }, hist, iscr, &rr);
    }
    // first rows and sizes of the candidates, fetched now (in flight while the band is classified
    // and re-scored) and used when publishing
    if (listed) {
#pragma unroll
      for (int j = 0; j < kCandCap / NT; ++j) {
        const int i = tid + j * NT;
        if (i < n_c) { const int c = cidl[i]; co[j] = a.offsets[(size_t)bg * (C + 1) + c]; ce[j] = a.offsets[(size_t)bg * (C + 1) + c + 1]; }
      }
    }
    // ---- in / band / out
    const double that = (double)f32_from_order_key(thr);
    const double hi = that + 2.0 * delta, lo = that - 2.0 * delta;
    // the band goes to a bitmap and, while it has at most kSmallBand members, straight to a list
    // in LDS (in no particular order); a longer band is listed from the bitmap in ascending id
    int nin = 0;
    auto classify = [&](int c, uint32_t k) {
      if (k == 0u) return;
      const double v = (double)f32_from_order_key(k);
      if (v > hi) { atomicOr(&bits[c >> 5], 1u << (c & 31)); ++nin; }
      else if (v >= lo) {
        atomicOr(&bbits[c >> 5], 1u << (c & 31));
        const int p = atomicAdd(&sh_i[7], 1);
        if (p < kSmallBand) band_lds[p] = c;
      }
    };
    if (listed) for (int i = tid; i < n_c; i += NT) classify(cidl[i], ckey[i]);
    else visit_keys(classify);
    const int n_in = block_isum<NT>(nin, iscr);          // includes a barrier
    const int need = k_eff - n_in;
    int n_band = sh_i[7];
    int32_t* band = band_lds;
    if (n_band > kSmallBand) {
      const int perw = (W32 + NT - 1) / NT;
      const int w0 = min(W32, tid * perw), w1 = min(W32, w0 + perw);
      int nb = 0;
      for (int w = w0; w < w1; ++w) nb += __popc(bbits[w]);
      int pos = block_exclusive_scan<NT>(nb, iscr, &n_band);
      band = a.band_ids + (size_t)bh * C;
      for (int w = w0; w < w1; ++w) {
        uint32_t m = bbits[w];
        while (m) { const int bit = __ffs(m) - 1; m &= m - 1; band[pos++] = w * 32 + bit; }
      }
      __syncthreads();
    }
    // (a band listed in LDS is read through band_lds itself: through the generic pointer the
    // reads would be flat loads, which wait for every global load in flight)
    if (need >= n_band) {
      if (n_band <= kSmallBand) {
        for (int i = tid; i < n_band; i += NT) { const int c = band_lds[i]; atomicOr(&bits[c >> 5], 1u << (c & 31)); }
      } else {
        for (int i = tid; i < n_band; i += NT) { const int c = band[i]; atomicOr(&bits[c >> 5], 1u << (c & 31)); }
      }
    } else if (n_band <= kSmallBand) {
      // canonical scores, one wave per band cluster: the lanes form the 128 exact products (two
      // each) in a row of LDS scratch (the publish arrays, free until publishing), then lane 0
      // adds them in ascending coordinate order -- the roundings of canonical_score_row.  Then
      // one wave ranks by (-sigma, id).
      static_assert((NT / 64) * kD * 8 <= 2 * kCandCap * 4, "a row of fp64 products per wave");
      static_assert(kSmallBand * 8 <= kFullCap * 4, "the band's score keys");
      double* prow = (wv < 8 ? reinterpret_cast<double*>(rl_off) : reinterpret_cast<double*>(rl_sz)) + (wv & 7) * kD;
      uint64_t* bk = reinterpret_cast<uint64_t*>(tfull);
      for (int j = wv; j < n_band; j += NT / 64) {
        const T* m = mu + (size_t)band_lds[j] * kD + 2 * lane;
        prow[2 * lane] = qd[2 * lane] * (double)St<T>::f(m[0]);
        prow[2 * lane + 1] = qd[2 * lane + 1] * (double)St<T>::f(m[1]);
        wave_lds_sync();
        if (lane == 0) {
          double acc = 0.0;
#pragma unroll 16
          for (int e = 0; e < kD; ++e) acc = acc + prow[e];
          bk[j] = f64_order_key(acc);
        }
        wave_lds_sync();
      }
      __syncthreads();
      if (wv == 0) {
        const bool live = lane < n_band;
        const int c = live ? band_lds[lane] : 0;
        const uint64_t key = live ? bk[lane] : 0ull;
        int rank = 0;
        for (int j = 0; j < n_band; ++j) {
          const uint64_t kj = bk[j];
          rank += (kj > key) || (kj == key && band_lds[j] < c);
        }
        if (live && rank < need) atomicOr(&bits[c >> 5], 1u << (c & 31));
      }
    } else {
      uint64_t* bkey = a.band_key + (size_t)bh * C;
      for (int i = tid; i < n_band; i += NT)
        bkey[i] = f64_order_key(canonical_score_row<T>(qd, mu + (size_t)band[i] * kD));
      __syncthreads();
      int rem2;
      const uint64_t t64 = block_radix_select<NT, uint64_t>(n_band, need, [&](int i) { return bkey[i]; }, hist, iscr, &rem2);
      // above the threshold: in; equal to it: the lowest ids (band order) fill the rest
      const int per2 = (n_band + NT - 1) / NT;
      const int i0 = min(n_band, tid * per2), i1 = min(n_band, i0 + per2);
      int neq = 0;
      for (int i = i0; i < i1; ++i) neq += (bkey[i] == t64);
      int tot_eq;
      int rk = block_exclusive_scan<NT>(neq, iscr, &tot_eq);
      for (int i = i0; i < i1; ++i) {
        const uint64_t kk = bkey[i];
        bool take = kk > t64;
        if (kk == t64) { take = rk < rem2; ++rk; }
        if (take) { const int c = band[i]; atomicOr(&bits[c >> 5], 1u << (c & 31)); }
      }
    }
  }
  __syncthreads();

  int k_zone = reuse ? n_reused_ne : k_eff;
  if (EXT && a.bounded) {
    // the k_eff selected clusters (the canonical top k_eff) with score keys and error terms (the
    // summary, candidate, histogram and publish arrays are free until publishing, which rebuilds
    // them); zo packs (score key, id) so that a larger value comes first in the order (-score, id)
    uint64_t* zo = reinterpret_cast<uint64_t*>(skey);
    int* zi = sid;
    float* ze = reinterpret_cast<float*>(rl_off);      // err
    float* zl = reinterpret_cast<float*>(ckey);        // lo
    float* za = reinterpret_cast<float*>(cidl);        // a
    float* zv = reinterpret_cast<float*>(hist);        // a V_c + w u V_c
    float* zt = reinterpret_cast<float*>(rl_sz);       // T(j): err summed over the clusters after the first j
    const int32_t* szg = a.sizes + (size_t)bg * C;
    const float* rdg = a.radius + (size_t)bg * C;
    const float* vng = a.vnorm + (size_t)bg * C;
    {
      const int perw = (W32 + NT - 1) / NT;
      const int w0 = min(W32, tid * perw), w1 = min(W32, w0 + perw);
      int n = 0;
      for (int w = w0; w < w1; ++w) n += __popc(bits[w]);
      int tot;
      int p = block_exclusive_scan<NT>(n, iscr, &tot);
      for (int w = w0; w < w1; ++w) {
        uint32_t m = bits[w];
        while (m) { zi[p++] = w * 32 + __ffs(m) - 1; m &= m - 1; }
      }
    }
    __syncthreads();
    float rmax = 0.f;                                  // largest radius of a non-empty cluster
    // the list's terms: every load of an entry issued before the first is used
    for (int i0 = 0; i0 < k_eff; i0 += 2 * NT) {
      int c[2];
      uint32_t kk[2];
      float nn[2], rr[2], vv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        c[u] = zi[min(i0 + u * NT + tid, k_eff - 1)];
        kk[u] = keys[c[u]]; nn[u] = (float)szg[c[u]]; rr[u] = rdg[c[u]]; vv[u] = vng[c[u]];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * NT + tid;
        if (i < k_eff) {
          const BTerms t = bound_terms(kk[u], nn[u], rr[u], vv[u]);
          zo[i] = ((uint64_t)kk[u] << 32) | (uint32_t)(0xffffffffu - (uint32_t)c[u]);
          ze[i] = t.err; zl[i] = t.lo; za[i] = t.ea; zv[i] = t.eav;
          rmax = fmaxf(rmax, rr[u]);
        }
      }
    }
    // the terms of the non-empty clusters outside the list, summed directly in one pass (a
    // difference of totals would cancel); loads unconditional (indices clamped), then masked
    float so = 0.f, slo = 0.f, sa_o = 0.f, sv_o = 0.f;
    for (int j0 = 0; j0 < KPT; j0 += 8) {
      uint32_t kk[8];
      float nn[8], rr[8], vv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = min((j0 + i) * NT + tid, C - 1);
        kk[i] = keys[c]; nn[i] = (float)szg[c]; rr[i] = rdg[c]; vv[i] = vng[c];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = (j0 + i) * NT + tid;
        const bool live = c < C && kk[i] != 0u && !((bits[min(c, C - 1) >> 5] >> (c & 31)) & 1u);
        if (live) {
          const BTerms t = bound_terms(kk[i], nn[i], rr[i], vv[i]);
          so += t.err; slo += t.lo; sa_o += t.ea; sv_o += t.eav;
          rmax = fmaxf(rmax, rr[i]);
        }
      }
    }
    float* red = reinterpret_cast<float*>(tfull);      // reduction scratch (free here)
    const float slo_o = slo;                           // lo outside the list (this thread's part)
    __syncthreads();                                   // the list's terms are visible
    for (int i = tid; i < k_eff; i += NT) slo += zl[i];
    float tot2[2] = {so, slo};
    block_sums_max<NT, 2>(tot2, rmax, red);
    const float e_out = tot2[0], b_lo = tot2[1], r_hi = rmax;
    const float lim = a.eps * b_lo;
    constexpr int EPT = kBoundedMaxTopK / NT;           // list entries per thread
    static_assert(EPT * NT == kBoundedMaxTopK && 2 * kBoundedMaxTopK <= kSumCap, "the bounded list's layout");
    // kf = the smallest zone size j whose first clusters in the order (-fp32 score, id) leave an
    // error sum T(j) <= eps * (sum of every lo); the cap k_eff when none does
    int kf = k_eff;
    if (k_eff > 0) {
      // ---- the list sorted: ranks (runs of 64 ranked in their waves, merged by binary search),
      // then every array permuted to them through registers
      uint64_t kv[EPT];
      int rk[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) { const int i = e * NT + tid; kv[e] = i < k_eff ? zo[i] : 0ull; }
      block_rank_desc<NT, EPT, true>(k_eff, kv, rk, [](uint64_t x, uint64_t y) { return x > y; },
                                     [&](int p, uint64_t k) { zo[p] = k; }, [&](int p) { return zo[p]; },
                                     [&](int p) { return zo[p]; });
      float pe[EPT], pl[EPT], pa[EPT], pv[EPT];
      int pc[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = min(e * NT + tid, k_eff - 1);
        pe[e] = ze[i]; pl[e] = zl[i]; pa[e] = za[i]; pv[e] = zv[i]; pc[e] = zi[i];
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        if (e * NT + tid < k_eff) {
          const int r = rk[e];
          zo[r] = kv[e]; ze[r] = pe[e]; zl[r] = pl[e]; za[r] = pa[e]; zv[r] = pv[e]; zi[r] = pc[e];
        }
      }
      __syncthreads();
      // ---- T(j) = e_out + the err of positions j .. k_eff - 1: thread t sums positions
      // k_eff - 1 - (t EPT + e), e < EPT, and an exclusive scan adds those of the threads before
      float loc[EPT], run = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int p = k_eff - 1 - (tid * EPT + e);
        run += p >= 0 ? ze[p] : 0.f;
        loc[e] = run;
      }
      float tot;
      const float before = block_exclusive_scan_f<NT>(run, fred, &tot);
      int kb = k_eff;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int p = k_eff - 1 - (tid * EPT + e);
        if (p >= 0) {
          const float t = e_out + (before + loc[e]);
          zt[p] = t;
          if (t <= lim) kb = min(kb, p);
        }
      }
      kf = (int)-block_max<NT>(-(float)kb, fred);      // includes barriers: zt is visible
    }
    // ---- certification: kf is the decision the canonical fp64 terms give when A(kf) <= eps and
    // A(kf - 1) > eps hold for every value within the fp32 error of the terms and sums.  The fp32
    // order's prefixes are the canonical ones up to clusters whose fp32 scores lie within 2 delta
    // of the boundary: the canonical first j hold positions [0, L_j), lie within [0, U_j) and
    // leave out U_j - j of the band [L_j, U_j), so T_canonical(j) lies between T(U_j) plus U_j - j
    // times the band's smallest err and T(U_j) plus U_j - j times its largest.
    bool cert = !EXACT;
    int zL = kf, zU = kf;                              // the band at the zone's boundary
    if (!EXACT && k_eff > 0) {
      auto sc_at = [&](int p) { return (double)f32_from_order_key((uint32_t)(zo[p] >> 32)); };
      auto t_at = [&](int p) { return p < k_eff ? (double)zt[p] : (double)e_out; };
      auto len_L = [&](int j) {
        if (j <= 0 || j >= k_eff) return j;
        const double s = sc_at(j) + 2.0 * delta;
        int L = j;
        while (L > 0 && sc_at(L - 1) <= s) --L;
        return L;
      };
      auto len_U = [&](int j) {
        if (j <= 0 || j >= k_eff) return j;
        const double s = sc_at(j - 1) - 2.0 * delta;
        int U = j;
        while (U < k_eff && sc_at(U) >= s) ++U;
        return U;
      };
      auto t_bound = [&](int j, bool upper) {
        const int L = len_L(j), U = len_U(j);
        float m = upper ? 0.f : INFINITY;
        for (int p = L; p < U; ++p) m = upper ? fmaxf(m, ze[p]) : fminf(m, ze[p]);
        return t_at(U) + (U > j ? (double)(U - j) * (double)m : 0.0);
      };
      // relative error budgets (u = 2^-24): the weights' exponent is off by scale delta from the
      // scores plus the roundings of scale s - m* and of the exponential's argument; x = scale |q|
      // r carries |q|'s rounding into expm1 and exp(-x); each term adds a few roundings, and each
      // sum at most one per addition on its longest path.  Doubled, plus an absolute allowance for
      // terms that underflow.
      const double u32 = 5.9604644775390625e-08, sc = (double)a.scale;
      const double amax = sc * ((double)qv * (1.0 + 1.0 / 1024) * (double)mxn * (1.0 + 1.0 / 1024) + delta);
      // e^y - 1 <= y (1 + y) for 0 <= y <= 1/2 (the series' tail is below y^2 e^y / 2)
      const double yw = sc * delta + 6.0 * u32 * amax + 4.0 * u32;
      const double rw = yw * (1.0 + yw) + 2.0 * u32;
      const double xh = sc * (double)qv * (double)r_hi * (1.0 + 1.0 / 1024);
      const double rx = (kD + 8) * u32;
      const double depth = (double)(KPT + 2 * EPT + 64) * u32;
      const double rT = 2.0 * (rw + (1.0 + xh) * rx + 12.0 * u32 + depth);
      const double rD = 2.0 * (rw + xh * rx + 2.0 * u32 * xh + 6.0 * u32 + depth);
      const double tiny = (double)n_ne * 0x1p-100;
      const double tauT = tiny * ((double)__expf((float)fmin(xh, 80.0)) * 1.01 + 1.0) * (1.0 + 3.0 * (double)b_vall);
      const double Dlo = (double)b_lo * (1.0 - rD) - tiny, Dhi = (double)b_lo * (1.0 + rD) + tiny;
      const double eps = (double)a.eps;
      cert = yw <= 0.5 && xh < 80.0 && Dlo > 0.0 && isfinite((double)b_lo) && isfinite((double)e_out);
      if (cert && kf < k_eff) {                       // A(kf) <= eps
        const double hiA = (t_bound(kf, true) * (1.0 + rT) + tauT) / Dlo;
        cert = isfinite(hiA) && hiA * (1.0 + 1e-9) < eps;
      }
      if (cert && kf > 0) {                           // A(kf - 1) > eps
        const double loA = (t_bound(kf - 1, false) * (1.0 - rT) - tauT) / Dhi;
        cert = loA * (1.0 - 1e-9) > eps;
      }
      if (cert) { zL = len_L(kf); zU = len_U(kf); }
    }
    if constexpr (!EXACT) {
      // an uncertified head leaves its outputs to the second launch
      if (tid == 0) a.bnd_redo[bh] = cert ? 0 : 1;
      if (!cert) return;
    }
    if (cert) {
      if (kf < k_eff) {
        // the zone: positions [0, zL), and the best kf - zL of the band [zL, zU) by (-canonical
        // score, id)
        for (int w = tid; w < W32; w += NT) bits[w] = 0u;
        __syncthreads();
        for (int p = tid; p < zL; p += NT) { const int c = zi[p]; atomicOr(&bits[c >> 5], 1u << (c & 31)); }
        if (zU > zL) {
          uint64_t* bkey = a.band_key + (size_t)bh * C;
          for (int p = zL + tid; p < zU; p += NT)
            bkey[p - zL] = f64_order_key(canonical_score_row<T>(qd, mu + (size_t)zi[p] * kD));
          __syncthreads();
          const int nb = zU - zL, need = kf - zL;
          for (int p = zL + tid; p < zU; p += NT) {
            const CanonKey me{bkey[p - zL], zi[p]};
            int r = 0;
            for (int j = 0; j < nb; ++j) r += canon_gt(CanonKey{bkey[j], zi[zL + j]}, me) ? 1 : 0;
            if (r < need) { const int c = zi[p]; atomicOr(&bits[c >> 5], 1u << (c & 31)); }
          }
        }
        __syncthreads();
      }
      k_zone = kf;
    } else if constexpr (EXACT) {
      // ---- the second launch: the decision in fp64
      k_zone = bounded_zone_fp64<T, NT>(
          (gbl_ptr<const uint32_t>)keys, (gbl_ptr<const T>)mu, (gbl_ptr<const int32_t>)szg,
          (gbl_ptr<const float>)rdg, (gbl_ptr<const float>)vng, (double)b_vall, (double)a.scale, (double)a.u,
          (double)a.eps, C, W32, k_eff, (lds_ptr<const double>)qd, (lds_ptr<const int>)zi, (lds_ptr<uint64_t>)zo,
          (lds_ptr<int>)(sid + kBoundedMaxTopK), (lds_ptr<uint32_t>)bits, (lds_ptr<double>)dscr,
          (lds_ptr<float>)fred);
      if (tid == 0 && a.bnd_fallback) atomicAdd(a.bnd_fallback, 1u);
    }
    // sums over the estimated clusters (outside the zone) for the bound after attention: the
    // clusters outside the list, plus the list entries the zone left out
    float s3[3] = {sa_o, sv_o, slo_o};
    for (int i = tid; i < k_eff; i += NT) {
      const int c = zi[i];
      if ((bits[c >> 5] >> (c & 31)) & 1u) continue;
      s3[0] += za[i]; s3[1] += zv[i]; s3[2] += zl[i];
    }
    float unused = 0.f;
    block_sums_max<NT, 3>(s3, unused, red);
    if (tid == 0) {
      float* bd = a.bnd + (size_t)bh * 4;
      bd[0] = b_mstar; bd[1] = s3[0]; bd[2] = s3[1]; bd[3] = s3[2];
      if (a.k_used) a.k_used[bh] = k_zone;
    }
    fast_pub = false;
  }

  // ---- publish, in ascending id: sel_ids and the head's list (id, first k_perm row, first
  // token after the steady zone, score key), padded to top_k; then, for every token workgroup
  // of the attention kernel, the list entry that holds its first retrieved token
  {
    const int K = a.top_k, S = a.att_split;
    const bool lists = !(EXT && a.refresh);   // refresh: sel_ids only (attention may read the lists)
    // ascending retrieved ids (LDS when they fit); on the candidate path each retrieved
    // candidate also drops its prefetched first row, size and key at its rank
    int32_t* rl = K <= kSumCap ? sid : a.band_ids + (size_t)bh * C;
    const int perw = (W32 + NT - 1) / NT;
    const int w0 = min(W32, tid * perw), w1 = min(W32, w0 + perw);
    int n = 0;
    for (int w = w0; w < w1; ++w) n += __popc(bits[w]);
    int tot;
    int p = block_exclusive_scan<NT>(n, iscr, &tot);
    if (fast_pub) {
      int* wpre = reinterpret_cast<int*>(bbits);      // the band bitmap is no longer needed
      for (int w = w0; w < w1; ++w) { wpre[w] = p; p += __popc(bits[w]); }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kCandCap / NT; ++j) {
        const int i = tid + j * NT;
        if (i < sh_i[2]) {
          const int c = cidl[i];
          const uint32_t wb = bits[c >> 5];
          if ((wb >> (c & 31)) & 1u) {
            const int r = wpre[c >> 5] + __popc(wb & ((1u << (c & 31)) - 1u));
            sid[r] = c; skey[r] = ckey[i]; rl_off[r] = co[j]; rl_sz[r] = ce[j] - co[j];
          }
        }
      }
    } else {
      for (int w = w0; w < w1; ++w) {
        uint32_t m = bits[w];
        while (m) { const int c = w * 32 + __ffs(m) - 1; m &= m - 1; rl[p++] = c; }
      }
    }
    tot = min(tot, K);
    __syncthreads();
    const int32_t* off = a.offsets + (size_t)bg * (C + 1);
    int32_t* out = a.sel_ids ? a.sel_ids + (size_t)bh * K : nullptr;
    const size_t lb = (size_t)bh * K, pb = (size_t)bh * (K + 1);
    int32_t* bounds = a.att_bounds + (size_t)bh * S;
    // token total first when the list takes several rounds
    int64_t ntok = a.NS;
    const int chunk = NT * kPubPT;
    if (tot > chunk) {
      int sum = 0;
      for (int i = tid; i < tot; i += NT) { const int c = rl[i]; sum += off[c + 1] - off[c]; }
      ntok += block_isum<NT>(sum, iscr);
    }
    int t_run = a.NS;
    for (int base = 0; base < tot; base += chunk) {
      const int i0 = base + tid * kPubPT;
      int c_[kPubPT], r_[kPubPT], z_[kPubPT];
      uint32_t k_[kPubPT];
      int ssum = 0;
#pragma unroll
      for (int u = 0; u < kPubPT; ++u) {
        const int i = i0 + u;
        c_[u] = 0; r_[u] = 0; z_[u] = 0; k_[u] = 0u;
        if (i < tot) {
          if (fast_pub) {
            c_[u] = sid[i]; r_[u] = rl_off[i]; z_[u] = rl_sz[i]; k_[u] = skey[i];
          } else {
            c_[u] = rl[i];
            r_[u] = off[c_[u]];
            z_[u] = off[c_[u] + 1] - r_[u];
            k_[u] = keys[c_[u]];
          }
          ssum += z_[u];
        }
      }
      int csum;
      int t = t_run + block_exclusive_scan<NT>(ssum, iscr, &csum);
      if (tot <= chunk) ntok = (int64_t)a.NS + csum;
      // token workgroup x covers [floor(x ntok / S), floor((x+1) ntok / S)); its first retrieved
      // token is u_x = max(that start, NS), and its entry the last one whose first token is
      // <= u_x.  u_x >= p holds for every x when p <= NS, else for x >= ceil(p S / ntok), so
      // entry i (tokens [t_i, t_i + size)) is the entry of x in [x_first(t_i), x_first(t_i +
      // size)), the last entry also of every later x
      auto x_first = [&](int p) -> int {
        return p <= a.NS ? 0 : (int)min<int64_t>(S, ((int64_t)p * S + ntok - 1) / ntok);
      };
#pragma unroll
      for (int u = 0; u < kPubPT; ++u) {
        const int i = i0 + u;
        if (i < tot) {
          if (out) out[i] = c_[u];
          if (lists) {
            a.hl_cid[lb + i] = c_[u];
            a.hl_row[lb + i] = r_[u];
            a.hl_pre[pb + i] = t;
            a.hl_key[lb + i] = k_[u];
            const int x1 = i == tot - 1 ? S : x_first(t + z_[u]);
            for (int x = x_first(t); x < x1; ++x) bounds[x] = i;
          }
          t += z_[u];
        }
      }
      t_run += csum;
    }
    for (int i = tot + tid; i < K; i += NT) {
      if (out) out[i] = -1;
      if (lists) { a.hl_cid[lb + i] = 0; a.hl_row[lb + i] = 0; a.hl_key[lb + i] = 0u; a.hl_pre[pb + i] = (int)ntok; }
    }
    if (!lists) return;
    if (tid == 0) a.hl_pre[pb + K] = (int)ntok;
    if (tot == 0) for (int x = tid; x < S; x += NT) bounds[x] = 0;
  }
  if (tid == 0) a.all_sel[bh] = k_zone == n_ne ? 1 : 0;
}

// ============================================================================ k_attend
constexpr int kAttThreads = 256;
constexpr int kAttStage = 512;      // row-map entries staged in LDS at a time

// Rows per lane group per pass (a lane group is 16 lanes sharing a row, lane&15 owns 8 dims).
template <typename T> struct AttRows { static constexpr int R = 4; };
template <> struct AttRows<float> { static constexpr int R = 2; };

// Online softmax state of one lane group.
template <int G>
struct OState {
  float m[G], den[G], num[G][8];
  __device__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY; den[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) num[h][e] = 0.f;
    }
  }
  // fold R rows with logits l (-inf = absent), denominator weights wd and packed values v
  template <int R, typename P>
  __device__ void add(const float (&l)[R][G], const float (&wd)[R], const P (&v)[R]) {
    float mx[G], sc[G];
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = m[h];
#pragma unroll
      for (int i = 0; i < R; ++i) mx[h] = fmaxf(mx[h], l[i][h]);
      any |= mx[h] != -INFINITY;
      sc[h] = (m[h] == -INFINITY || mx[h] == -INFINITY) ? 0.f : __expf(m[h] - mx[h]);
      den[h] *= sc[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) num[h][e] *= sc[h];
      m[h] = mx[h];
    }
    if (!any) return;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float vf[8];
      v[i].unpack(vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = l[i][h] == -INFINITY ? 0.f : __expf(l[i][h] - mx[h]);
        den[h] += wd[i] * p;
#pragma unroll
        for (int e = 0; e < 8; ++e) num[h][e] += p * vf[e];
      }
    }
  }
};

// Combine the 16 lane-group states of the block and write one partial per head to `slot`.
template <int G>
__device__ void write_partial(OState<G>& st, size_t slot, float* md_out, float* num_out,
                              float* sh_m, float* sh_den, float* sh_num) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      const float om = __shfl_xor(st.m[h], x);
      const float mx = fmaxf(st.m[h], om);
      const float s0 = st.m[h] == -INFINITY ? 0.f : __expf(st.m[h] - mx);
      const float s1 = om == -INFINITY ? 0.f : __expf(om - mx);
      st.den[h] = st.den[h] * s0 + __shfl_xor(st.den[h], x) * s1;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.num[h][e] = st.num[h][e] * s0 + __shfl_xor(st.num[h][e], x) * s1;
      st.m[h] = mx;
    }
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sh_num[(w * G + h) * kD + 8 * lr + e] = st.num[h][e];
      if (lr == 0) { sh_m[w * G + h] = st.m[h]; sh_den[w * G + h] = st.den[h]; }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kD; i += kAttThreads) {
    const int h = i / kD;
    float mx = -INFINITY;
    for (int ww = 0; ww < 4; ++ww) mx = fmaxf(mx, sh_m[ww * G + h]);
    float s = 0.f;
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = sh_m[ww * G + h];
      if (mw != -INFINITY) s += __expf(mw - mx) * sh_num[ww * G * kD + i];
    }
    num_out[slot * G * kD + i] = s;
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float mx = -INFINITY;
    for (int ww = 0; ww < 4; ++ww) mx = fmaxf(mx, sh_m[ww * G + h]);
    float d = 0.f;
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = sh_m[ww * G + h];
      if (mw != -INFINITY) d += __expf(mw - mx) * sh_den[ww * G + h];
    }
    md_out[(slot * G + h) * 2] = mx;
    md_out[(slot * G + h) * 2 + 1] = d;
  }
}


// Max over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15), in every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));   // quad [1,0,3,2]
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));   // quad [2,3,0,1]
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));  // row half mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));  // row mirror
  return v;
}

// Scores of a query against 16 key rows on MFMA: A = the query (row 0; rows 1-15 zero), B = the
// keys (column = token).  Lane (lr = lane & 15, lg = lane >> 4) supplies token lr; the result
// lane (lr, lg = 0) holds the score of token lr in register 0.
template <typename T> struct QkTile;
template <> struct QkTile<uint16_t> {
  bf16x8_t q[4], k[4];
  // MFMA step s consumes dims 32 s + 8 lg .. +8 of both operands (64 contiguous bytes per row
  // across the four lanes of a lane column)
  __device__ void load_q(const uint16_t* qh, int lr, int lg) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (lr == 0) q[s] = *reinterpret_cast<const bf16x8_t*>(qh + 32 * s + 8 * lg);
      else q[s] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  __device__ void load_k(const uint16_t* row, int lg) {
#pragma unroll
    for (int s = 0; s < 4; ++s) k[s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(row + 32 * s + 8 * lg));
  }
  __device__ void zero_k() {
#pragma unroll
    for (int s = 0; s < 4; ++s) k[s] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }
  __device__ f32x4_t scores() const {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[s], k[s], acc, 0, 0, 0);
    return acc;
  }
};
template <> struct QkTile<float> {
  float q[32];
  u32x4_t k[8];
  // MFMA step 4 j + e consumes dim 16 j + 4 lg + e of both operands
  __device__ void load_q(const float* qh, int lr, int lg) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (lr == 0) v = *reinterpret_cast<const u32x4_t*>(qh + 16 * j + 4 * lg);
      q[4 * j] = __uint_as_float(v.x); q[4 * j + 1] = __uint_as_float(v.y);
      q[4 * j + 2] = __uint_as_float(v.z); q[4 * j + 3] = __uint_as_float(v.w);
    }
  }
  __device__ void load_k(const float* row, int lg) {
#pragma unroll
    for (int j = 0; j < 8; ++j) k[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + 16 * j + 4 * lg));
  }
  __device__ void zero_k() {
#pragma unroll
    for (int j = 0; j < 8; ++j) k[j] = u32x4_t{0u, 0u, 0u, 0u};
  }
  __device__ f32x4_t scores() const {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q[4 * j], __uint_as_float(k[j].x), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q[4 * j + 1], __uint_as_float(k[j].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q[4 * j + 2], __uint_as_float(k[j].z), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(q[4 * j + 3], __uint_as_float(k[j].w), acc, 0, 0, 0);
    }
    return acc;
  }
};

// grid (B*Hq * (S + Sc)): workgroup (bh, s).  For s < S it attends exactly over tokens
// [s n_tok / S, (s+1) n_tok / S) of query head bh's list: the steady zone, then the rows of the
// head's retrieved clusters in ascending cluster id.  Workgroup S + j folds the estimation terms
// of entries [64 j, 64 j + 64) of the head's retrieved list into a partial the merge subtracts.
//
// Token workgroups map their tokens to rows through the list (first token of every entry, in
// LDS, binary-searched per token), then each wave takes 16-token steps (key and value rows
// loaded non-temporally: 1M tokens 35.6 -> 34.1 us, batch 16 118.9 -> 110.1 us): the query is
// scored against the 16 key rows on MFMA, the running max comes from a DPP row reduction, and the
// probabilities go through a 64-byte LDS slot of the wave to the lanes that hold the value rows
// (lane (lr, lg) holds dims 8 lr .. 8 lr + 7 of tokens 4 i + lg), which accumulate P V.
template <typename T, bool PG>
__global__ __launch_bounds__(kAttThreads) void k_attend(DecodeArgs a) {
  constexpr int R = AttRows<T>::R;
  constexpr int PASS = 16 * R;                 // corrections: 4 waves x 4 lane groups x R rows
  __shared__ float sh_m[4], sh_den[4];
  __shared__ float sh_num[4 * kD];
  __shared__ uint32_t sh_ent[kAttStage];       // token -> row | host (bit 29) | steady (30) | valid (31)
  __shared__ int spre[kAttStage + 1];          // first token of list entries e_cur + x
  __shared__ int srow[kAttStage];              // first k_perm row of list entries e_cur + x
  __shared__ float sh_p[4][16];
  __shared__ int sh_next;
  const int items = a.att_items, S = a.att_split, K = a.top_k;
  // group-fastest numbering: every workgroup of a KV group's heads runs on the group's XCD
  const int BG = a.B * a.Hkv, j = blockIdx.x / BG, bgx = blockIdx.x - j * BG;
  const int hix = j % a.G, s = j / a.G;
  const int bh = bgx * a.G + hix;
  const int b = bh / a.Hq, h = bh - b * a.Hq, bg = b * a.Hkv + h / a.G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int NS = a.NS;
  const int32_t* pre = a.hl_pre + (size_t)bh * (K + 1);
  OState<1> st;
  st.init();
  if (s < S) {
    const int ntok = pre[K];
    int e_cur = K > 0 ? a.att_bounds[(size_t)bh * S + s] : 0;
    const int t0 = (int)(((int64_t)s * ntok) / S), t1 = (int)(((int64_t)(s + 1) * ntok) / S);
    const int32_t* rowl = a.hl_row + (size_t)bh * K;
    QkTile<T> qk;
    qk.load_q(static_cast<const T*>(a.q) + (size_t)bh * kD, lr, lg);
    // retrieved rows: the index's cluster-major copy, or with a wave buffer the block pool (cache
    // and execution buffer) and, for blocks it could not stage, the copy in host memory
    const T* hk = static_cast<const T*>(a.k_perm) + (size_t)bg * a.Nc * kD;
    const T* hv = static_cast<const T*>(a.v_perm) + (size_t)bg * a.Nc * kD;
    const T* kp = PG ? static_cast<const T*>(a.pool_k) : hk;
    const T* vp = PG ? static_cast<const T*>(a.pool_v) : hv;
    const int32_t* wloc = PG ? a.wb_loc + (size_t)bg * a.wb_nblk : nullptr;
    const T* ks = static_cast<const T*>(a.k_steady) + (size_t)bg * NS * kD;
    const T* vs = static_cast<const T*>(a.v_steady) + (size_t)bg * NS * kD;
    for (int z0 = t0; z0 < t1; z0 += kAttStage) {
      const int z1 = min(t1, z0 + kAttStage);
      if (z0 > t0) __syncthreads();            // the previous chunk's map is no longer read
      for (int t = z0 + tid; t < min(z1, NS); t += kAttThreads) sh_ent[t - z0] = (uint32_t)t | (3u << 30);
      const int u0 = max(z0, NS);
      if (u0 < z1) {
        // the at most z1 - u0 <= kAttStage entries that hold tokens [u0, z1) start at e_cur
        for (int x = tid; x <= kAttStage; x += kAttThreads) {
          const int e = e_cur + x;
          spre[x] = e <= K ? pre[e] : ntok;
          if (x < kAttStage) srow[x] = e < K ? rowl[e] : 0;
        }
        __syncthreads();
        for (int t = u0 + tid; t < z1; t += kAttThreads) {
          int lo = 0, hi = kAttStage;            // spre[lo] <= t < spre[hi]
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (spre[mid] <= t) lo = mid; else hi = mid;
          }
          const int row = srow[lo] + (t - spre[lo]);
          uint32_t ent = (uint32_t)row | (1u << 31);
          if constexpr (PG) {
            const int loc = wloc[row >> 4];        // pool block, or -1: read from host memory
            ent = loc >= 0 ? ((uint32_t)(loc * kWbBlock + (row & (kWbBlock - 1))) | (1u << 31)) : (ent | (1u << 29));
          }
          sh_ent[t - z0] = ent;
          if (t == z1 - 1) sh_next = e_cur + lo;
        }
      }
      __syncthreads();
      if (u0 < z1) e_cur = sh_next;
      const int nsteps = (z1 - z0 + 15) >> 4;
      for (int j = w; j < nsteps; j += 4) {
        const int base = z0 + 16 * j;
        // key row of token base + lr (MFMA operand), value rows of tokens base + 4 i + lg
        const int tk = base + lr;
        const uint32_t eK = tk < z1 ? sh_ent[tk - z0] : 0u;
        if ((eK >> 31) != 0u)
          qk.load_k((((eK >> 30) & 1u) ? ks : (PG && ((eK >> 29) & 1u)) ? hk : kp) + (size_t)(eK & 0x1fffffffu) * kD, lg);
        else qk.zero_k();
        Piece<T> vr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tv = base + 4 * i + lg;
          const uint32_t eV = tv < z1 ? sh_ent[tv - z0] : 0u;
          if ((eV >> 31) != 0u)
            vr[i].load_nt((((eV >> 30) & 1u) ? vs : (PG && ((eV >> 29) & 1u)) ? hv : vp) + (size_t)(eV & 0x1fffffffu) * kD + 8 * lr);
          else vr[i].zero();
        }
        const f32x4_t acc = qk.scores();
        const float sc = (lg == 0 && (eK >> 31) != 0u) ? acc[0] * a.scale : -INFINITY;
        const float hm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row16_max(sc)), 0));
        const float mn = fmaxf(st.m[0], hm);
        const float alpha = (st.m[0] == mn) ? 1.f : __expf(st.m[0] - mn);
        const bool rescale = st.m[0] != mn;
        st.m[0] = mn;
        wave_lds_sync();
        if (lg == 0) sh_p[w][lr] = sc == -INFINITY ? 0.f : __expf(sc - mn);
        wave_lds_sync();
        if (rescale) {
          st.den[0] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) st.num[0][e] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = sh_p[w][4 * i + lg];
          float vf[8];
          vr[i].unpack(vf);
          st.den[0] += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) st.num[0][e] += p * vf[e];
        }
      }
    }
  } else {
    const int e0 = (s - S) * kCorrEntries, e1 = min(K, e0 + kCorrEntries);
    const T* sv = static_cast<const T*>(a.sv) + (size_t)bg * a.C * kD;
    const size_t lb = (size_t)bh * K;
    for (int c0 = e0; c0 < e1; c0 += PASS) {
      Piece<T> vr[R];
      float wd[R], l[R][1];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int e = c0 + w * (4 * R) + 4 * i + lg;
        const bool live = e < e1;
        const int c = live ? a.hl_cid[lb + e] : 0;
        const uint32_t key = live ? a.hl_key[lb + e] : 0u;
        wd[i] = live ? (float)(pre[e + 1] - pre[e]) : 0.f;
        if (key != 0u) vr[i].load(sv + (size_t)c * kD + 8 * lr);
        else vr[i].zero();
        l[i][0] = key != 0u ? f32_from_order_key(key) * a.scale : -INFINITY;
      }
      st.template add<R>(l, wd, vr);
    }
  }
  write_partial<1>(st, (size_t)bh * items + s, a.att_md, a.att_num, sh_m, sh_den, sh_num);
}

// ============================================================================ k_merge
// One workgroup per query head, with no block barrier (except for the bound of the bounded
// decode): wave w takes columns [128 w / NW, 128 (w + 1) / NW) of every partial, as QPW float4
// quads; lane (q, sl) = q + QPW sl folds quad q of partials sl, sl + SPW, sl + 2 SPW, ...  Every
// wave reads all the (m, den) pairs itself (64 per lane round), forms the largest partial max and
// the denominator with wave reductions, and hands each lane the merge factors of its partials by
// lane shuffles; the slices are summed by a butterfly over the slice bits.  The smallest of 128
// and 256 threads whose first round of loads covers every partial (at most 48 or 96), else 1024
// (128K tokens, batch 1, 43 partials per head: 4.28 us with 256 threads, 4.11 with 128).  The
// pairs of the first kMergeMd rounds and the numerators of the first kMergeU partials per lane
// are requested together, before anything is known; any further partials are read in later
// rounds.
constexpr int kMergeThreadsSmall = 128, kMergeThreadsFew = 256, kMergeThreadsMany = 1024;
constexpr int kMergeMd = 4;
constexpr int kMergeU = 12;
template <int NT> struct MergeShape {
  static constexpr int NW = NT / 64, QPW = 32 / NW, SPW = 64 / QPW;
  static constexpr int kFirst = SPW * kMergeU;     // partials the first round of numerators covers
};

// out = num / den, lse = M + log(den) with M the largest partial max, den = sum_p s_p f_p den_p,
// num = sum_p s_p f_p num_p, f_p = exp(m_p - M): estimation tiles (s = +1), exact splits (+1),
// retrieved-cluster corrections (s = -1).  A head that retrieved every non-empty cluster takes
// only its exact splits.
template <int NT>
__global__ __launch_bounds__(NT) void k_merge(DecodeArgs a) {
  using SH = MergeShape<NT>;
  constexpr int NW = SH::NW, QPW = SH::QPW, SPW = SH::SPW;
  __shared__ float sh_red[2 * NW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sl = lane / QPW, quad = w * QPW + (lane - sl * QPW);
  const int bh = head_of_block(a, blockIdx.x);
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int G = a.G, g = h / G, hi = h - g * G, bg = b * a.Hkv + g;
  // partials in order: PE estimation tiles, S token workgroups, PC correction workgroups; when
  // the head's all-retrieved flag is set the estimation and correction partials are dead (not
  // used, whatever they hold)
  const int all_sel = a.all_sel[bh];
  const int PE = a.est_blocks_g;
  const int S = a.att_split, items = a.att_items;
  const int P = PE + items;
  auto md_of = [&](int p) -> const float2* {
    if (p < PE) return reinterpret_cast<const float2*>(a.est_md + (((size_t)bg * a.est_blocks_g + p) * G + hi) * 2);
    return reinterpret_cast<const float2*>(a.att_md + ((size_t)bh * items + (p - PE)) * 2);
  };
  const float* est_col = a.est_num + ((size_t)bg * a.est_blocks_g * G + hi) * kD + 4 * quad;
  const float* att_col = a.att_num + (size_t)bh * items * kD + 4 * quad;
  // quad of partial p; past P the last partial is read and unused
  auto num_col = [&](int p) -> float4 {
    p = min(p, P - 1);
    const float* q = p < PE ? est_col + (size_t)p * G * kD : att_col + (size_t)(p - PE) * kD;
    return *reinterpret_cast<const float4*>(q);
  };
  float2 md[kMergeMd];
#pragma unroll
  for (int u = 0; u < kMergeMd; ++u) md[u] = *md_of(min(lane + 64 * u, P - 1));
  float4 v[kMergeU];
#pragma unroll
  for (int j = 0; j < kMergeU; ++j) v[j] = num_col(sl + SPW * j);
  const bool use_est = all_sel == 0;
  auto live = [&](int p, float den) { return den > 0.f && (use_est || (p >= PE && p < PE + S)); };
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < kMergeMd; ++u) {
    const int p = lane + 64 * u;
    if (p < PE + S && live(p, md[u].y)) mx = fmaxf(mx, md[u].x);
  }
  for (int p = lane + 64 * kMergeMd; p < PE + S; p += 64) {
    const float2 m2 = *md_of(p);
    if (live(p, m2.y)) mx = fmaxf(mx, m2.x);
  }
  const float M = wave_max(mx);
  // merge factor of a live partial, negated for the corrections; 0 for a dead one
  auto factor_of = [&](int p, float2 m2) -> float {
    if (!live(p, m2.y)) return 0.f;
    const float f = __expf(m2.x - M);
    return p >= PE + S ? -f : f;
  };
  float f[kMergeMd];
  float dn = 0.f, dx = 0.f;                      // dx: the exact partials (bounded decode)
#pragma unroll
  for (int u = 0; u < kMergeMd; ++u) {
    const int p = lane + 64 * u;
    f[u] = p < P ? factor_of(p, md[u]) : 0.f;
    if (f[u] != 0.f) {
      dn += f[u] * md[u].y;
      if (p >= PE && p < PE + S) dx += f[u] * md[u].y;
    }
  }
  for (int p = lane + 64 * kMergeMd; p < P; p += 64) {
    const float2 m2 = *md_of(p);
    const float fp = factor_of(p, m2);
    if (fp != 0.f) {
      dn += fp * m2.y;
      if (p >= PE && p < PE + S) dx += fp * m2.y;
    }
  }
  const float den = wave_sum(dn);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fold = [&](float fp, const float4& x) {
    if (fp != 0.f) { acc.x += fp * x.x; acc.y += fp * x.y; acc.z += fp * x.z; acc.w += fp * x.w; }
  };
  // the first round: partial p = sl + SPW j takes its factor from lane p mod 64 of round p / 64
  // (the same round for every lane of the wave, since SPW divides 64)
#pragma unroll
  for (int j = 0; j < kMergeU; ++j) {
    const int p = sl + SPW * j;
    const int u = (SPW * j) >> 6;
    float fp;
    if (u < kMergeMd) {
      float fu = f[0];
#pragma unroll
      for (int uu = 1; uu < kMergeMd; ++uu) if (uu == u) fu = f[uu];
      fp = __shfl(fu, p & 63);
    } else {
      fp = p < P ? factor_of(p, *md_of(p)) : 0.f;
    }
    if (p < P) fold(fp, v[j]);
  }
  // any further partials, kMergeU per lane a round, their factors recomputed from their pairs
  for (int p0 = SPW * kMergeU; p0 < P; p0 += SPW * kMergeU) {
#pragma unroll
    for (int j = 0; j < kMergeU; ++j) v[j] = num_col(p0 + sl + SPW * j);
#pragma unroll
    for (int j = 0; j < kMergeU; ++j) {
      const int p = p0 + sl + SPW * j;
      if (p < P) fold(factor_of(p, *md_of(p)), v[j]);
    }
  }
  // sum over the slices (lanes q + QPW sl, sl = 0 .. SPW - 1)
#pragma unroll
  for (int m = QPW; m < 64; m <<= 1) {
    acc.x += __shfl_xor(acc.x, m); acc.y += __shfl_xor(acc.y, m);
    acc.z += __shfl_xor(acc.z, m); acc.w += __shfl_xor(acc.w, m);
  }
  float o2 = 0.f;
  if (sl == 0) {
    const float4 o = make_float4(acc.x / den, acc.y / den, acc.z / den, acc.w / den);
    *reinterpret_cast<float4*>(a.out + (size_t)bh * kD + 4 * quad) = o;
    o2 = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
  }
  if (tid == 0 && a.lse) a.lse[bh] = M + __logf(den);
  if (a.bounded) {
    // error bound of the output: (sum a (V_c + |o|) + w u V_c) / (D_x + sum lo) over the estimated
    // clusters, their sums taken by the select in the frame m*, D_x = the exact partials' total
    const float Dx = wave_sum(dx);
    const float ow = wave_sum(o2);
    if (lane == 0) sh_red[w] = ow;
    __syncthreads();
    if (tid == 0 && a.err_bound) {
      float on2 = 0.f;
      for (int i = 0; i < NW; ++i) on2 += sh_red[i];
      const float on = sqrtf(on2);
      const float* bd = a.bnd + (size_t)bh * 4;
      float e = 0.f;
      if (bd[1] != 0.f || bd[2] != 0.f || bd[3] != 0.f) {
        const float fb = __expf(bd[0] - M);
        e = (bd[2] + on * bd[1]) * fb / (Dx + bd[3] * fb);
      }
      a.err_bound[bh] = e;
    }
  }
}

// ============================================================================ launcher
// the select: one workgroup per query head, followed by the estimation workgroups (none for a
// refresh, which only selects); half-size blocks where select_half_blocks says so; the gated,
// refresh and bounded modes in their own instantiation, so that the plain decode's kernel
// carries none of their code
template <typename T>
static void launch_select(const DecodeArgs& a, hipStream_t s) {
  const int BH = a.B * a.Hq;
  const unsigned grid = (unsigned)BH + (a.refresh ? 0u : (unsigned)(a.B * a.Hkv) * (unsigned)a.est_blocks_g);
  const bool ext = a.gated || a.refresh || a.bounded;
  const size_t lds = (size_t)a.W32 * 8;
  if (select_half_blocks(BH, a.C)) {
    if (ext) hipLaunchKernelGGL((k_select<T, kSelThreadsMany, 1>), dim3(grid), dim3(kSelThreadsMany), lds, s, a);
    else hipLaunchKernelGGL((k_select<T, kSelThreadsMany, 0>), dim3(grid), dim3(kSelThreadsMany), lds, s, a);
    if (a.bounded) hipLaunchKernelGGL((k_select<T, kSelThreadsMany, 2>), dim3(BH), dim3(kSelThreadsMany), lds, s, a);
  } else {
    if (ext) hipLaunchKernelGGL((k_select<T, kSelThreadsFew, 1>), dim3(grid), dim3(kSelThreadsFew), lds, s, a);
    else hipLaunchKernelGGL((k_select<T, kSelThreadsFew, 0>), dim3(grid), dim3(kSelThreadsFew), lds, s, a);
    if (a.bounded) hipLaunchKernelGGL((k_select<T, kSelThreadsFew, 2>), dim3(BH), dim3(kSelThreadsFew), lds, s, a);
  }
}

template <typename T, int G>
static hipError_t launch_groups(const DecodeArgs& a, hipStream_t s) {
  const int BG = a.B * a.Hkv, BH = a.B * a.Hq;
  const int merge_parts = a.est_blocks_g + a.att_items;
  const int merge_nt = merge_parts <= MergeShape<kMergeThreadsSmall>::kFirst ? kMergeThreadsSmall
                     : merge_parts <= MergeShape<kMergeThreadsFew>::kFirst ? kMergeThreadsFew : kMergeThreadsMany;
  hipError_t e;
  prof_begin(WI_STAGE_SCORE, s);
  // (while profiling with repeats, every kernel runs prof_reps() times: each is idempotent, and
  // repeat r may read a copy of the index at other addresses: prof_args)
  for (int r = 0; r < prof_reps(); ++r) {
    hipLaunchKernelGGL((k_score<T, G>), dim3(std::max(1, a.tiles_g), BG), dim3(kScoreThreads), 0, s, prof_args(a, r));
  }
  prof_end(WI_STAGE_SCORE, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin(WI_STAGE_SELECT, s);
  for (int r = 0; r < prof_reps(); ++r) launch_select<T>(prof_args(a, r), s);
  prof_end(WI_STAGE_SELECT, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.paged && (e = launch_wb_resolve(a, s)) != hipSuccess) return e;   // blocks of the zones
  prof_begin(WI_STAGE_ATTEND, s);
  for (int r = 0; r < prof_reps(); ++r) {
    if (a.paged)
      hipLaunchKernelGGL((k_attend<T, true>), dim3((unsigned)BH * (unsigned)a.att_items), dim3(kAttThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k_attend<T, false>), dim3((unsigned)BH * (unsigned)a.att_items), dim3(kAttThreads), 0, s, prof_args(a, r));
  }
  prof_end(WI_STAGE_ATTEND, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin(WI_STAGE_MERGE, s);
  for (int r = 0; r < prof_reps(); ++r) {
    if (merge_nt == kMergeThreadsSmall) hipLaunchKernelGGL(k_merge<kMergeThreadsSmall>, dim3(BH), dim3(kMergeThreadsSmall), 0, s, a);
    else if (merge_nt == kMergeThreadsFew) hipLaunchKernelGGL(k_merge<kMergeThreadsFew>, dim3(BH), dim3(kMergeThreadsFew), 0, s, a);
    else hipLaunchKernelGGL(k_merge<kMergeThreadsMany>, dim3(BH), dim3(kMergeThreadsMany), 0, s, a);
  }
  prof_end(WI_STAGE_MERGE, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_refresh_t(const DecodeArgs& a, hipStream_t s) {
  prof_begin(WI_STAGE_REFRESH, s);
  for (int r = 0; r < prof_reps(); ++r) launch_select<T>(a, s);
  prof_end(WI_STAGE_REFRESH, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: return launch_groups<T, 1>(a, s);
    case 2: return launch_groups<T, 2>(a, s);
    case 4: return launch_groups<T, 4>(a, s);
    case 8: return launch_groups<T, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t set_select_lds() {
  static bool attr_set = false;
  if (!attr_set) {
    // the select kernel's two cluster bitmaps (2 * ceil(C / 32) words) live in dynamic LDS
    const void* fns[12] = {reinterpret_cast<const void*>(k_select<float, kSelThreadsFew, 0>),
                           reinterpret_cast<const void*>(k_select<float, kSelThreadsMany, 0>),
                           reinterpret_cast<const void*>(k_select<uint16_t, kSelThreadsFew, 0>),
                           reinterpret_cast<const void*>(k_select<uint16_t, kSelThreadsMany, 0>),
                           reinterpret_cast<const void*>(k_select<float, kSelThreadsFew, 1>),
                           reinterpret_cast<const void*>(k_select<float, kSelThreadsMany, 1>),
                           reinterpret_cast<const void*>(k_select<uint16_t, kSelThreadsFew, 1>),
                           reinterpret_cast<const void*>(k_select<uint16_t, kSelThreadsMany, 1>),
                           reinterpret_cast<const void*>(k_select<float, kSelThreadsFew, 2>),
                           reinterpret_cast<const void*>(k_select<float, kSelThreadsMany, 2>),
                           reinterpret_cast<const void*>(k_select<uint16_t, kSelThreadsFew, 2>),
                           reinterpret_cast<const void*>(k_select<uint16_t, kSelThreadsMany, 2>)};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kSelectBitmapLds);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  return hipSuccess;
}

hipError_t launch_decode(const wi_decode_params& p, const DecodeArgs& a, hipStream_t s) {
  const hipError_t e = set_select_lds();
  if (e != hipSuccess) return e;
  return p.dtype == WI_BF16 ? launch_decode_t<uint16_t>(a, s) : launch_decode_t<float>(a, s);
}

hipError_t launch_refresh(const wi_decode_params& p, const DecodeArgs& a, hipStream_t s) {
  const hipError_t e = set_select_lds();
  if (e != hipSuccess) return e;
  return p.dtype == WI_BF16 ? launch_refresh_t<uint16_t>(a, s) : launch_refresh_t<float>(a, s);
}

}  // namespace wi

