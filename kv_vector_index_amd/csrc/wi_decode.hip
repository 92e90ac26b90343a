// Wave-index decode step on gfx950: score + estimate -> select -> work lists -> exact attention
// -> LSE merge.
//
// Method: RetroInfer's tripartite attention (technical summary, gist.science Spanish page,
// section 2.A items 1-3; Arabic page section 2.a).  Per query head, the steady zone (sinks and
// local window) and the retrieval zone (all tokens of the top_k clusters by <q, mu_c>) are
// attended exactly; every other non-empty cluster contributes n_c * exp(s_c) to the softmax
// denominator and n_c * exp(s_c) * SV_c / n_c to the numerator; the partial softmax states are
// merged with log-sum-exp.
//
// The estimation is computed over *all* non-empty clusters in the same pass that scores them
// (mu and SV stream together, before the selection is known), and the terms of the retrieved
// clusters are subtracted at the merge: sum over E = sum over all - sum over R.  The subtracted
// terms never exceed the exact mass of the same tokens (exp is convex, so n_c exp(mean logit) is
// at most the sum of the members' exp(logit)), so the cancellation costs O(eps_fp32) relative to
// the merged denominator.  When a head retrieves every non-empty cluster both terms are dropped.
//
// Kernels (one stream, in order; no kernel waits on another block of its own grid):
//   k_score_est  grid (ceil(C/128), B*Hkv): MFMA scores of the KV group's query heads against 128
//                centroids (one pass over mu serves all heads of the group), fp32 centroid norms,
//                and the tile's estimation partial per head from SV and the sizes.
//   k_select     grid (B*Hq): exact top-k per head (radix select on the fp32 scores, canonical
//                fp64 re-scoring of the certified uncertainty band, ties to the lower id).
//   k_union      grid (B*Hkv): union of the group's selections with a per-head mask, token
//                prefix sums and chunk starts.
//   k_attend     grid (S, B*Hkv): per KV group, items are 128-token chunks of steady + retrieved
//                rows (each row loaded once and used by every head of the group that selected
//                it) and 128-entry correction items (the retrieved clusters' estimation terms).
//   k_merge      grid (B*Hq): log-sum-exp merge of the head's partials into out and lse.
#include "wi_device.h"
#include "wi_internal.h"

namespace wi {

constexpr int kScoreThreads = 256;

// ============================================================================ k_score_est
template <typename T, int G>
__global__ __launch_bounds__(kScoreThreads) void k_score_est(DecodeArgs a) {
  __shared__ float sh_s[G][kEstTile];       // logits (scaled), -inf for empty clusters
  __shared__ float sh_w[G][kEstTile];       // exp(logit - m)
  __shared__ float sh_n[kEstTile];          // cluster sizes
  __shared__ float sh_m[G], sh_den[G];
  __shared__ float sh_num[4][G][kD];
  const int tile = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int C = a.C;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int cbase = tile * kEstTile + w * 32;
  const T* mu = static_cast<const T*>(a.mu) + (size_t)bg * C * kD;
  const T* sv = static_cast<const T*>(a.sv) + ((size_t)bg * C + (size_t)tile * kEstTile) * kD;
  const int32_t* szs = a.sizes + (size_t)bg * C;
  const T* qg = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)g * G) * kD;
  const int nrows = min(kEstTile, C - tile * kEstTile);

  // value sums of the tile: thread (w, lane) owns rows w + 4i and dims 2*lane, 2*lane+1.  The
  // loads are issued first; they do not depend on the scores.
  float2 svv[kEstTile / 4];
#pragma unroll
  for (int i = 0; i < kEstTile / 4; ++i) {
    const int r = w + 4 * i;
    svv[i] = make_float2(0.f, 0.f);
    if (r < nrows) {
      if constexpr (sizeof(T) == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(sv + (size_t)r * kD + 2 * lane);
        svv[i] = make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
      } else {
        svv[i] = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(sv) + (size_t)r * kD + 2 * lane);
      }
    }
  }
  if (tid < kEstTile) sh_n[tid] = tid < nrows ? (float)szs[tile * kEstTile + tid] : 0.f;

  if constexpr (sizeof(T) == 2) {
    // A = query heads (row = lane&15), B = centroids (column = lane&15).  Along k, lane group lg
    // owns dims [32*lg, 32*lg+32); MFMA step s consumes dims 32*lg + 8s .. +8 on both operands.
    bf16x8_t qa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (lr < G) qa[s] = *reinterpret_cast<const bf16x8_t*>(qg + (size_t)lr * kD + 32 * lg + 8 * s);
      else qa[s] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int c = cbase + 16 * t + lr;
      bf16x8_t mb[4];
      int sz = 0;
      if (c < C) {
        sz = szs[c];
        const T* row = mu + (size_t)c * kD + 32 * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) mb[s] = *reinterpret_cast<const bf16x8_t*>(row + 8 * s);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) mb[s] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], mb[s], acc, 0, 0, 0);
      float n2 = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float x = (float)mb[s][e]; n2 += x * x; }
      n2 += __shfl_xor(n2, 16);
      n2 += __shfl_xor(n2, 32);
      const int cl = w * 32 + 16 * t + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * lg + r;
        if (h < G) {
          if (c < C) a.scores[((size_t)b * a.Hq + (size_t)g * G + h) * C + c] = acc[r];
          sh_s[h][cl] = (c < C && sz > 0) ? acc[r] * a.scale : -INFINITY;
        }
      }
      if (lg == 0 && c < C) a.mu_norm[(size_t)bg * C + c] = sqrtf(n2);
    }
  } else {
    // fp32: 16x16x4 MFMA, 32 steps; step s consumes dim 32*lg + s on both operands.
    float qa[32];
#pragma unroll
    for (int s = 0; s < 32; s += 8) {
      float tmp[8];
      if (lr < G) St<float>::load8(reinterpret_cast<const float*>(qg) + (size_t)lr * kD + 32 * lg + s, tmp);
      else for (int e = 0; e < 8; ++e) tmp[e] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) qa[s + e] = tmp[e];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int c = cbase + 16 * t + lr;
      float mb[32];
      int sz = 0;
      if (c < C) {
        sz = szs[c];
        const float* row = reinterpret_cast<const float*>(mu) + (size_t)c * kD + 32 * lg;
#pragma unroll
        for (int s = 0; s < 32; s += 8) {
          float tmp[8];
          St<float>::load8(row + s, tmp);
#pragma unroll
          for (int e = 0; e < 8; ++e) mb[s + e] = tmp[e];
        }
      } else {
#pragma unroll
        for (int s = 0; s < 32; ++s) mb[s] = 0.f;
      }
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 32; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[s], mb[s], acc, 0, 0, 0);
      float n2 = 0.f;
#pragma unroll
      for (int s = 0; s < 32; ++s) n2 += mb[s] * mb[s];
      n2 += __shfl_xor(n2, 16);
      n2 += __shfl_xor(n2, 32);
      const int cl = w * 32 + 16 * t + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * lg + r;
        if (h < G) {
          if (c < C) a.scores[((size_t)b * a.Hq + (size_t)g * G + h) * C + c] = acc[r];
          sh_s[h][cl] = (c < C && sz > 0) ? acc[r] * a.scale : -INFINITY;
        }
      }
      if (lg == 0 && c < C) a.mu_norm[(size_t)bg * C + c] = sqrtf(n2);
    }
  }
  __syncthreads();

  // estimation partial of the tile: m_h = max logit, den_h = sum n_c w, num_h = sum w SV_c
  for (int h = w; h < G; h += kScoreThreads / 64) {
    const float x0 = sh_s[h][lane], x1 = sh_s[h][lane + 64];
    const float m = wave_max(fmaxf(x0, x1));
    const float w0 = x0 == -INFINITY ? 0.f : __expf(x0 - m);
    const float w1 = x1 == -INFINITY ? 0.f : __expf(x1 - m);
    sh_w[h][lane] = w0;
    sh_w[h][lane + 64] = w1;
    const float dn = wave_sum(w0 * sh_n[lane] + w1 * sh_n[lane + 64]);
    if (lane == 0) { sh_m[h] = m; sh_den[h] = dn; }
  }
  __syncthreads();
  float2 acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = make_float2(0.f, 0.f);
#pragma unroll
  for (int i = 0; i < kEstTile / 4; ++i) {
    const int r = w + 4 * i;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float wt = sh_w[h][r];
      acc[h].x += wt * svv[i].x;
      acc[h].y += wt * svv[i].y;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    sh_num[w][h][2 * lane] = acc[h].x;
    sh_num[w][h][2 * lane + 1] = acc[h].y;
  }
  __syncthreads();
  const size_t slot = (size_t)bg * a.est_tiles_g + tile;
  for (int i = tid; i < G * kD; i += kScoreThreads) {
    const int h = i / kD, d = i - h * kD;
    a.est_num[(slot * G + h) * kD + d] = sh_num[0][h][d] + sh_num[1][h][d] + sh_num[2][h][d] + sh_num[3][h][d];
  }
  if (tid < G) {
    a.est_md[(slot * G + tid) * 2] = sh_m[tid];
    a.est_md[(slot * G + tid) * 2 + 1] = sh_den[tid];
  }
}

// ============================================================================ k_select
constexpr int kSelThreads = 512;
constexpr int kSmallBand = 64;      // bands up to one wave are resolved by direct ranking

// Radix bin of the k-th largest key: threads 0..255 own the bins in descending order, so an
// inclusive scan over them gives suffix counts; the one bin with excl < rem <= incl is chosen.
__device__ __forceinline__ void radix_pick(const uint32_t* hist, int rem, int* scr, int* out_bin,
                                           int* out_above) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bin = 255 - tid;
  const int v = tid < 256 ? (int)hist[bin] : 0;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63 && w < 4) scr[w] = inc;
  __syncthreads();
  if (tid < 256) {
    int base = 0;
    for (int i = 0; i < w; ++i) base += scr[i];
    const int incl = base + inc, excl = incl - v;
    if (excl < rem && rem <= incl) { *out_bin = bin; *out_above = excl; }
  }
  __syncthreads();
}

// Threshold key of the k-th largest of n keys (1 <= k <= n): afterwards exactly k - *rem_out keys
// are strictly greater than the returned key and at least *rem_out keys equal it.
template <typename K, typename Get>
__device__ K block_radix_select(int n, int k, Get get, uint32_t* hist, int* scr, int* rem_out) {
  K prefix = 0, mask = 0;
  int rem = k;
  for (int shift = (int)sizeof(K) * 8 - 8; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const K key = get(i);
      if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    radix_pick(hist, rem, scr, scr + 8, scr + 9);
    prefix |= (K)scr[8] << shift;
    rem -= scr[9];
    mask |= (K)255 << shift;
  }
  *rem_out = rem;
  return prefix;
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

template <typename T>
__global__ __launch_bounds__(kSelThreads) void k_select(DecodeArgs a) {
  extern __shared__ uint32_t dyn[];           // bitmap [W32], then keys [C] when they fit
  __shared__ uint32_t hist[256];
  __shared__ int iscr[48];
  __shared__ float fscr[32];
  __shared__ double qd[kD];
  __shared__ int band_lds[kSmallBand];

  const int tid = threadIdx.x, NT = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int G = a.G, g = h / G, bg = b * a.Hkv + g;
  const int C = a.C, W32 = a.W32;
  uint32_t* bits = dyn;
  const bool keys_in_lds = (size_t)C * 4 + (size_t)W32 * 4 <= 65536;
  uint32_t* keys = keys_in_lds ? dyn + W32 : a.keys32 + (size_t)bh * C;
  const int32_t* off = a.offsets + (size_t)bg * (C + 1);
  const int32_t* sizes = a.sizes + (size_t)bg * C;
  const float* sc = a.scores + (size_t)bh * C;
  const float* mnorm = a.mu_norm + (size_t)bg * C;
  const T* qh = static_cast<const T*>(a.q) + (size_t)bh * kD;
  const T* mu = static_cast<const T*>(a.mu) + (size_t)bg * C * kD;

  float qv = 0.f;
  if (tid < kD) { qv = St<T>::f(qh[tid]); qd[tid] = (double)qv; }
  const float qn = sqrtf(block_sum(qv * qv, fscr));

  for (int w = tid; w < W32; w += NT) bits[w] = 0u;
  // order keys (0 marks an empty cluster), non-empty count, largest centroid norm
  int cnt = 0;
  float mxn = 0.f;
  for (int base = tid; base < C; base += 4 * NT) {
    int sz[4];
    float s[4], nm[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = base + u * NT;
      sz[u] = 0; s[u] = 0.f; nm[u] = 0.f;
      if (c < C) { sz[u] = sizes[c]; s[u] = sc[c]; nm[u] = mnorm[c]; }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = base + u * NT;
      if (c < C) {
        uint32_t key = 0u;
        if (sz[u] > 0) { ++cnt; mxn = fmaxf(mxn, nm[u]); key = f32_order_key(s[u]); }
        keys[c] = key;
      }
    }
  }
  const int n_ne = block_isum(cnt, iscr);
  mxn = block_max(mxn, fscr);
  const int k_eff = min(a.top_k, n_ne);
  __syncthreads();

  if (k_eff > 0 && k_eff == n_ne) {
    for (int c = tid; c < C; c += NT)
      if (keys[c] != 0u) atomicOr(&bits[c >> 5], 1u << (c & 31));
  } else if (k_eff > 0) {
    int rem;
    const uint32_t thr = block_radix_select<uint32_t>(C, k_eff, [&](int i) { return keys[i]; }, hist, iscr, &rem);
    // Certified band: |fp32 score - canonical fp64 score| <= delta for every cluster (fp32
    // accumulation of d exact-or-rounded products, doubled for an unspecified MFMA order).
    const double that = (double)f32_from_order_key(thr);
    const double delta = 2.0 * (kD + 2) * 5.9604644775390625e-08 * (double)qn * (1.0 + 1.0 / 1024) *
                             (double)mxn * (1.0 + 1.0 / 1024) + 1e-30;
    const double hi = that + 2.0 * delta, lo = that - 2.0 * delta;
    const int per = (C + NT - 1) / NT;
    const int c0 = min(C, tid * per), c1 = min(C, c0 + per);
    int nb = 0, nin = 0;
    for (int c = c0; c < c1; ++c) {
      const uint32_t key = keys[c];
      if (key == 0u) continue;
      const double v = (double)f32_from_order_key(key);
      if (v > hi) { atomicOr(&bits[c >> 5], 1u << (c & 31)); ++nin; }
      else if (v >= lo) ++nb;
    }
    int n_band;
    int pos = block_exclusive_scan(nb, iscr, &n_band);
    const int n_in = block_isum(nin, iscr);
    const int need = k_eff - n_in;
    int32_t* band = n_band <= kSmallBand ? band_lds : a.band_ids + (size_t)bh * C;
    for (int c = c0; c < c1; ++c) {
      const uint32_t key = keys[c];
      if (key == 0u) continue;
      const double v = (double)f32_from_order_key(key);
      if (!(v > hi) && v >= lo) band[pos++] = c;
    }
    __syncthreads();
    if (need >= n_band) {
      for (int i = tid; i < n_band; i += NT) { const int c = band[i]; atomicOr(&bits[c >> 5], 1u << (c & 31)); }
    } else if (n_band <= kSmallBand) {
      // one wave: rescore, then rank by (-sigma, id); the band is in ascending id order
      if (wv == 0) {
        const bool live = lane < n_band;
        const int c = live ? band[lane] : 0;
        const uint64_t key = live ? f64_order_key(canonical_score_row<T>(qd, mu + (size_t)c * kD)) : 0ull;
        int rank = 0;
        for (int j = 0; j < n_band; ++j) {
          const uint64_t kj = __shfl(key, j);
          rank += (kj > key) || (kj == key && j < lane);
        }
        if (live && rank < need) atomicOr(&bits[c >> 5], 1u << (c & 31));
      }
    } else {
      uint64_t* bkey = a.band_key + (size_t)bh * C;
      for (int i = tid; i < n_band; i += NT)
        bkey[i] = f64_order_key(canonical_score_row<T>(qd, mu + (size_t)band[i] * kD));
      __syncthreads();
      int rem2;
      const uint64_t t64 = block_radix_select<uint64_t>(n_band, need, [&](int i) { return bkey[i]; }, hist, iscr, &rem2);
      // above the threshold: in; equal to it: the lowest ids (band order) fill the rest
      const int per2 = (n_band + NT - 1) / NT;
      const int i0 = min(n_band, tid * per2), i1 = min(n_band, i0 + per2);
      int neq = 0;
      for (int i = i0; i < i1; ++i) neq += (bkey[i] == t64);
      int tot_eq;
      int r = block_exclusive_scan(neq, iscr, &tot_eq);
      for (int i = i0; i < i1; ++i) {
        const uint64_t kk = bkey[i];
        bool take = kk > t64;
        if (kk == t64) { take = r < rem2; ++r; }
        if (take) { const int c = band[i]; atomicOr(&bits[c >> 5], 1u << (c & 31)); }
      }
    }
  }
  __syncthreads();

  // publish the bitmap; ascending ids to sel_ids
  uint32_t* gbits = a.sel_bits + (size_t)bh * W32;
  for (int w = tid; w < W32; w += NT) gbits[w] = bits[w];
  if (a.sel_ids) {
    const int perw = (W32 + NT - 1) / NT;
    const int w0 = min(W32, tid * perw), w1 = min(W32, w0 + perw);
    int n = 0;
    for (int w = w0; w < w1; ++w) n += __popc(bits[w]);
    int tot;
    int p = block_exclusive_scan(n, iscr, &tot);
    int32_t* out = a.sel_ids + (size_t)bh * a.top_k;
    for (int w = w0; w < w1; ++w) {
      uint32_t m = bits[w];
      while (m) { const int bit = __ffs(m) - 1; m &= m - 1; if (p < a.top_k) out[p] = w * 32 + bit; ++p; }
    }
    for (int i = tot + tid; i < a.top_k; i += NT) out[i] = -1;
  }

  if (tid == 0) a.all_sel[bh] = (k_eff == n_ne) ? 1 : 0;
}

// ============================================================================ k_union
constexpr int kUnionThreads = 512;
constexpr int kUnionLds = 4096;

// Union of the selections of a KV group's query heads, in ascending cluster id, with the mask of
// the heads that selected each cluster; token prefix sums (the steady zone first) and the first
// entry of every 128-token chunk.
__global__ __launch_bounds__(kUnionThreads) void k_union(DecodeArgs a) {
  __shared__ int iscr[48];
  __shared__ int ucid_lds[kUnionLds];
  const int tid = threadIdx.x, NT = blockDim.x;
  const int bg = blockIdx.x;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int G = a.G, C = a.C, W32 = a.W32;
  const uint32_t* hb = a.sel_bits + ((size_t)b * a.Hq + (size_t)g * G) * W32;
  const int32_t* off = a.offsets + (size_t)bg * (C + 1);
  const int32_t* sizes = a.sizes + (size_t)bg * C;
  int32_t* cidg = a.wl_cid + (size_t)bg * a.Umax;
  int32_t* ucid = a.Umax <= kUnionLds ? ucid_lds : cidg;
  int32_t* umask = a.wl_mask + (size_t)bg * a.Umax;
  const int perw = (W32 + NT - 1) / NT;
  const int w0 = min(W32, tid * perw), w1 = min(W32, w0 + perw);
  int ne = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t u = 0u;
    for (int j = 0; j < G; ++j) u |= hb[(size_t)j * W32 + w];
    ne += __popc(u);
  }
  int n_entries;
  int e = block_exclusive_scan(ne, iscr, &n_entries);
  for (int w = w0; w < w1; ++w) {
    uint32_t hw[kMaxGroup];
    uint32_t u = 0u;
    for (int j = 0; j < G; ++j) { hw[j] = hb[(size_t)j * W32 + w]; u |= hw[j]; }
    while (u) {
      const int bit = __ffs(u) - 1;
      u &= u - 1;
      int m = 0;
      for (int j = 0; j < G; ++j) m |= (int)((hw[j] >> bit) & 1u) << j;
      ucid[e] = w * 32 + bit;
      umask[e] = m;
      ++e;
    }
  }
  __syncthreads();
  const int pe = (n_entries + NT - 1) / NT;
  const int e0 = min(n_entries, tid * pe), e1 = min(n_entries, e0 + pe);
  int nt = 0;
  for (int i = e0; i < e1; ++i) nt += sizes[ucid[i]];
  int n_utok;
  int t = block_exclusive_scan(nt, iscr, &n_utok);
  const int NS = a.NS;
  const int n_tok = NS + n_utok;
  int32_t* row0 = a.wl_row0 + (size_t)bg * a.Umax;
  int32_t* pre = a.wl_pre + (size_t)bg * (a.Umax + 1);
  int32_t* ce0 = a.chunk_e0 + (size_t)bg * a.max_chunks_g;
  for (int i = e0; i < e1; ++i) {
    const int c = ucid[i];
    const int r0 = off[c], sz = sizes[c];
    const int start = NS + t;
    row0[i] = r0;
    pre[i] = start;
    if (ucid != cidg) cidg[i] = c;
    // chunks whose first token falls inside this cluster's token range start at entry i
    for (int j = (start + kChunkTokens - 1) / kChunkTokens; j * kChunkTokens < start + sz; ++j) ce0[j] = i;
    t += sz;
  }
  for (int j = tid; j * kChunkTokens < min(NS, n_tok); j += NT) ce0[j] = 0;   // chunks in the steady zone
  if (tid == 0) {
    pre[n_entries] = n_tok;
    int32_t* gd = a.grp + (size_t)bg * 4;
    gd[0] = n_entries;
    gd[1] = n_tok;
    gd[2] = (n_tok + kChunkTokens - 1) / kChunkTokens;
    gd[3] = (n_entries + kEstTile - 1) / kEstTile;
  }
}

// ============================================================================ k_attend
constexpr int kAttThreads = 256;

// Rows of a work item: wave w owns rows w*32 + 4*i + (lane>>4), i = 0..7; lane&15 owns dims
// [8*(lane&15), +8).  Given per-row logits (identical across the 16 lanes of a row), the row
// values and a per-row weight of the denominator, form the item's partial softmax state per head
// (max logit m, den = sum wden e^(l-m), num = sum e^(l-m) v) and write it to `slot`.
template <int G>
__device__ __forceinline__ void finish_partial(const float (&l)[8][G], const float (&v)[8][8],
                                               const float (&wden)[8], size_t slot, const DecodeArgs& a,
                                               float* sh_m, float* sh_num, float* sh_den) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15;
  float M[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = l[0][h];
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, l[i][h]);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lane == 0) sh_m[w * G + h] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = sh_m[h];
    for (int ww = 1; ww < kAttThreads / 64; ++ww) m = fmaxf(m, sh_m[ww * G + h]);
    M[h] = m;
  }
  float den[G], num[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    den[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) num[h][e] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = (l[i][h] == -INFINITY) ? 0.f : __expf(l[i][h] - M[h]);
      den[h] += wden[i] * p;
#pragma unroll
      for (int e = 0; e < 8; ++e) num[h][e] += p * v[i][e];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    den[h] += __shfl_xor(den[h], 16);
    den[h] += __shfl_xor(den[h], 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      num[h][e] += __shfl_xor(num[h][e], 16);
      num[h][e] += __shfl_xor(num[h][e], 32);
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sh_num[(w * G + h) * kD + 8 * lr + e] = num[h][e];
      if (lr == 0) sh_den[w * G + h] = den[h];
    }
  }
  __syncthreads();
  float* pn = a.att_num + slot * G * kD;
  for (int i = threadIdx.x; i < G * kD; i += kAttThreads) {
    float s = 0.f;
    for (int ww = 0; ww < kAttThreads / 64; ++ww) s += sh_num[ww * G * kD + i];
    pn[i] = s;
  }
  if (threadIdx.x < G) {
    const int hh = threadIdx.x;
    float s = 0.f;
    for (int ww = 0; ww < kAttThreads / 64; ++ww) s += sh_den[ww * G + hh];
    a.att_md[(slot * G + hh) * 2 + 0] = M[hh];
    a.att_md[(slot * G + hh) * 2 + 1] = s;
  }
  __syncthreads();
}

// The estimation terms of the retrieved clusters (entries [128 ci, 128 ci + 128) of the group's
// union list), for the heads that retrieved each one; the merge subtracts them.
template <typename T, int G>
__device__ void corr_item(const DecodeArgs& a, int bg, int ci, int n_entries, size_t slot,
                          float* sh_m, float* sh_num, float* sh_den) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, rg = lane >> 4;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv, C = a.C;
  const int32_t* szs = a.sizes + (size_t)bg * C;
  const T* sv = static_cast<const T*>(a.sv) + (size_t)bg * C * kD;
  const int32_t* cid = a.wl_cid + (size_t)bg * a.Umax;
  const int32_t* msk = a.wl_mask + (size_t)bg * a.Umax;
  const size_t hbase = (size_t)b * a.Hq + (size_t)g * G;
  float l[8][G], v[8][8], wden[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = ci * kEstTile + w * 32 + 4 * i + rg;
    const bool live = e < n_entries;
    const int c = live ? cid[e] : 0;
    const int m = live ? msk[e] : 0;
    wden[i] = live ? (float)szs[c] : 0.f;
    if (live) St<T>::load8(sv + (size_t)c * kD + 8 * lr, v[i]);
    else for (int x = 0; x < 8; ++x) v[i][x] = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
      l[i][h] = ((m >> h) & 1) ? a.scores[(hbase + h) * C + c] * a.scale : -INFINITY;
  }
  finish_partial<G>(l, v, wden, slot, a, sh_m, sh_num, sh_den);
}

template <typename T, int G>
__device__ void attend_chunk(const DecodeArgs& a, int bg, int jl, int n_entries, int n_tok,
                             size_t slot, float* sh_m, float* sh_num, float* sh_den, int* sh_row,
                             int* sh_mask) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, rg = lane >> 4;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int NS = a.NS;
  const int t0 = jl * kChunkTokens;
  const int t1 = min(n_tok, t0 + kChunkTokens);
  const int32_t* row0 = a.wl_row0 + (size_t)bg * a.Umax;
  const int32_t* msk = a.wl_mask + (size_t)bg * a.Umax;
  const int32_t* pre = a.wl_pre + (size_t)bg * (a.Umax + 1);
  const int e0 = a.chunk_e0[(size_t)bg * a.max_chunks_g + jl];

  // token -> (row, head mask); row >= 0 indexes k_perm, row < 0 is steady row (-1 - row)
  for (int t = t0 + threadIdx.x; t < min(t1, NS); t += kAttThreads) {
    sh_row[t - t0] = -1 - t;
    sh_mask[t - t0] = (1 << G) - 1;
  }
  for (int e = e0 + threadIdx.x; e < n_entries; e += kAttThreads) {
    const int s = pre[e];
    if (s >= t1) break;
    const int s1 = pre[e + 1];
    const int r0 = row0[e], m = msk[e];
    for (int t = max(s, t0); t < min(s1, t1); ++t) { sh_row[t - t0] = r0 + (t - s); sh_mask[t - t0] = m; }
  }
  __syncthreads();

  const T* kp = static_cast<const T*>(a.k_perm) + (size_t)bg * a.Nc * kD;
  const T* vp = static_cast<const T*>(a.v_perm) + (size_t)bg * a.Nc * kD;
  const T* ks = static_cast<const T*>(a.k_steady) + (size_t)bg * NS * kD;
  const T* vs = static_cast<const T*>(a.v_steady) + (size_t)bg * NS * kD;
  const T* qg = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)g * G) * kD;

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) St<T>::load8(qg + (size_t)h * kD + 8 * lr, qf[h]);

  float kr[8][8], v[8][8], wden[8];
  int mk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = w * 32 + 4 * i + rg;
    const int t = t0 + r;
    wden[i] = 1.f;
    mk[i] = 0;
    if (t < t1) {
      const int row = sh_row[r];
      mk[i] = sh_mask[r];
      const T* kq = row >= 0 ? kp + (size_t)row * kD : ks + (size_t)(-1 - row) * kD;
      const T* vq = row >= 0 ? vp + (size_t)row * kD : vs + (size_t)(-1 - row) * kD;
      St<T>::load8(kq + 8 * lr, kr[i]);
      St<T>::load8(vq + 8 * lr, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { kr[i][e] = 0.f; v[i][e] = 0.f; }
    }
  }
  float l[8][G];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += qf[h][e] * kr[i][e];
      s += __shfl_xor(s, 8);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 1);
      l[i][h] = ((mk[i] >> h) & 1) ? s * a.scale : -INFINITY;
    }
  }
  finish_partial<G>(l, v, wden, slot, a, sh_m, sh_num, sh_den);
}

template <typename T, int G>
__global__ __launch_bounds__(kAttThreads) void k_attend(DecodeArgs a) {
  __shared__ float sh_m[4 * G];
  __shared__ float sh_den[4 * G];
  __shared__ float sh_num[4 * G * kD];
  __shared__ int sh_row[kChunkTokens];
  __shared__ int sh_mask[kChunkTokens];
  const int bg = blockIdx.y;
  const int32_t* gd = a.grp + (size_t)bg * 4;
  const int n_entries = gd[0], n_tok = gd[1], n_chunks = gd[2], n_corr = gd[3];
  for (int it = blockIdx.x; it < n_chunks + n_corr; it += gridDim.x) {
    const size_t slot = (size_t)bg * a.att_items_g + it;
    if (it < n_chunks)
      attend_chunk<T, G>(a, bg, it, n_entries, n_tok, slot, sh_m, sh_num, sh_den, sh_row, sh_mask);
    else
      corr_item<T, G>(a, bg, it - n_chunks, n_entries, slot, sh_m, sh_num, sh_den);
  }
}

// ============================================================================ k_merge
constexpr int kMergeThreads = 256;
constexpr int kMergeLds = 8192;

// out = num / den, lse = M + log(den) with M the largest partial max, den = sum_p s_p f_p den_p,
// num = sum_p s_p f_p num_p, f_p = exp(m_p - M): estimation tiles (s = +1), exact chunks (+1),
// retrieved-cluster corrections (s = -1).  A head that retrieved every non-empty cluster takes
// only its exact chunks.
__global__ __launch_bounds__(kMergeThreads) void k_merge(DecodeArgs a) {
  __shared__ float sh_f[kMergeLds];
  __shared__ float sh_red[32];
  __shared__ float4 sh_acc[kMergeThreads / 32][32];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int G = a.G, g = h / G, hi = h - g * G, bg = b * a.Hkv + g;
  const int32_t* gd = a.grp + (size_t)bg * 4;
  const int n_chunks = gd[2], n_corr = gd[3];
  const bool use_est = a.all_sel[bh] == 0;
  const int PE = use_est ? a.est_tiles_g : 0;
  const int PC = use_est ? n_corr : 0;
  const int P = PE + n_chunks + PC;
  // partial p: [0, PE) estimation tiles, [PE, PE + n_chunks) chunks, then corrections
  auto md_of = [&](int p) -> const float* {
    if (p < PE) return a.est_md + (((size_t)bg * a.est_tiles_g + p) * G + hi) * 2;
    return a.att_md + (((size_t)bg * a.att_items_g + (p - PE)) * G + hi) * 2;
  };
  auto num_of = [&](int p) -> const float* {
    if (p < PE) return a.est_num + (((size_t)bg * a.est_tiles_g + p) * G + hi) * kD;
    return a.att_num + (((size_t)bg * a.att_items_g + (p - PE)) * G + hi) * kD;
  };
  float mx = -INFINITY;
  for (int p = tid; p < PE + n_chunks; p += kMergeThreads) {
    const float2 md = *reinterpret_cast<const float2*>(md_of(p));
    if (md.y > 0.f) mx = fmaxf(mx, md.x);
  }
  const float M = block_max(mx, sh_red);
  const bool f_lds = P <= kMergeLds;
  float dn = 0.f;
  for (int p = tid; p < P; p += kMergeThreads) {
    const float2 md = *reinterpret_cast<const float2*>(md_of(p));
    float f = md.y > 0.f ? __expf(md.x - M) : 0.f;
    if (p >= PE + n_chunks) f = -f;
    if (f_lds) sh_f[p] = f;
    dn += f * md.y;
  }
  const float den = block_sum(dn, sh_red);
  __syncthreads();
  // numerators: 32 float4 columns cover the head's 128 dims; 8 replicas split the partials
  const int col = tid & 31, rep = tid >> 5;
  constexpr int R = kMergeThreads / 32;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = rep; p0 < P; p0 += 8 * R) {
    float4 v[8];
    float f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * R;
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      f[u] = 0.f;
      if (p < P) {
        v[u] = *reinterpret_cast<const float4*>(num_of(p) + 4 * col);
        if (f_lds) {
          f[u] = sh_f[p];
        } else {
          const float2 md = *reinterpret_cast<const float2*>(md_of(p));
          f[u] = md.y > 0.f ? __expf(md.x - M) : 0.f;
          if (p >= PE + n_chunks) f[u] = -f[u];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x += f[u] * v[u].x; acc.y += f[u] * v[u].y; acc.z += f[u] * v[u].z; acc.w += f[u] * v[u].w;
    }
  }
  sh_acc[rep][col] = acc;
  __syncthreads();
  if (tid < 32) {
    float4 s = sh_acc[0][tid];
    for (int r = 1; r < R; ++r) {
      const float4 t = sh_acc[r][tid];
      s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
    }
    *reinterpret_cast<float4*>(a.out + (size_t)bh * kD + 4 * tid) = make_float4(s.x / den, s.y / den, s.z / den, s.w / den);
  }
  if (tid == 0 && a.lse) a.lse[bh] = M + __logf(den);
}

// ============================================================================ launcher
template <typename T, int G>
static hipError_t launch_groups(const DecodeArgs& a, hipStream_t s) {
  const int BG = a.B * a.Hkv, BH = a.B * a.Hq;
  hipError_t e;
  if (a.C > 0) {
    prof_begin(WI_STAGE_SCORE, s);
    hipLaunchKernelGGL((k_score_est<T, G>), dim3(a.est_tiles_g, BG), dim3(kScoreThreads), 0, s, a);
    prof_end(WI_STAGE_SCORE, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const bool keys_in_lds = (size_t)a.C * 4 + (size_t)a.W32 * 4 <= 65536;
  const size_t dyn = (size_t)a.W32 * 4 + (keys_in_lds ? (size_t)a.C * 4 : 0);
  prof_begin(WI_STAGE_SELECT, s);
  hipLaunchKernelGGL(k_select<T>, dim3(BH), dim3(kSelThreads), dyn, s, a);
  hipLaunchKernelGGL(k_union, dim3(BG), dim3(kUnionThreads), 0, s, a);
  prof_end(WI_STAGE_SELECT, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int S = (int)std::max<int64_t>(1, std::min<int64_t>(a.att_items_g, ceil_div(1024, BG)));
  prof_begin(WI_STAGE_ATTEND, s);
  hipLaunchKernelGGL((k_attend<T, G>), dim3(S, BG), dim3(kAttThreads), 0, s, a);
  prof_end(WI_STAGE_ATTEND, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin(WI_STAGE_MERGE, s);
  hipLaunchKernelGGL(k_merge, dim3(BH), dim3(kMergeThreads), 0, s, a);
  prof_end(WI_STAGE_MERGE, s);
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

hipError_t launch_decode(const wi_decode_params& p, const DecodeArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_select<float>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 98304);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_select<uint16_t>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 98304);
    attr_set = true;
  }
  return p.dtype == WI_BF16 ? launch_decode_t<uint16_t>(a, s) : launch_decode_t<float>(a, s);
}

}  // namespace wi
