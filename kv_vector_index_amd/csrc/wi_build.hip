// Wave-index build on gfx950: segmented spherical k-means (RetroInfer technical summary,
// gist.science Spanish page sections 2.A item 2 and 3 "Clustering Segmentado"; Arabic page
// section 2.a), then the index buffers the decode step reads.
//
// Every decision is reproducible bit for bit: assignments are made on fp32 MFMA scores and every
// key whose top two scores are closer than the certified fp32 error band is re-decided with the
// canonical fp64 score (exact products, ascending coordinate order); cluster sums are fp64 in
// ascending token order; normalisation uses IEEE fp64 sqrt and division and rounds fp64 -> fp32
// -> bf16 with round-to-nearest-even.
//
// Kernels (one stream, in order):
//   k_prep      steady-zone copies, re-decision counter reset
//   k_init      per segment: SplitMix64-driven partial Fisher-Yates picks the seed rows;
//               directions = rounded unit seed keys
//   then `iters` times:
//     k_assign  MFMA keys x centroid directions (centroids staged in LDS, keys in registers)
//               with a fused running top-2 per key; uncertain keys go to a list, which a block
//               holding every centroid of its segment re-decides itself in fp64
//     k_rescore fp64 canonical argmax for the listed keys (centroids not resident in LDS)
//     k_csr     per segment: counts, offsets and a stable counting scatter -> sizes/offsets/perm
//     k_update2 (all but the last iteration) fp64 member sums -> new unit directions
//     k_final   (last iteration) mean keys, value sums, cluster-major K/V copies
#include <type_traits>

#include "wi_device.h"
#include "wi_internal.h"

namespace wi {

struct BuildArgs {
  const void* k;      // [BG, N, d]
  const void* v;
  void* mu;           // [BG, C, d]
  void* sv;
  int32_t* sizes;     // [BG, C]
  int32_t* offsets;   // [BG, C+1]
  int32_t* perm;      // [BG, Nc]
  void* kp;           // [BG, Nc, d]
  void* vp;
  void* ks;           // [BG, NS, d]
  void* vs;
  void* mhat;         // [BG, C, d] centroid directions (workspace)
  int32_t* assign;    // [BG, Nc] local cluster id per clustered token
  uint32_t* flag_cnt; // [iters]
  int32_t* flag_list; // [BG * Nc]
  int Hkv, N, sink, window, NS, lo, Nc, L, nseg, Cs, C, BG, iters;
  int seg0;           // segments [seg0, nseg) are built; the others are left as they are
  uint64_t seed;
};

__device__ __forceinline__ int seg_len_of(const BuildArgs& a, int s) { return min(a.L, a.Nc - s * a.L); }

// ============================================================================ k_prep
template <typename T>
__global__ __launch_bounds__(256) void k_prep(BuildArgs a) {
  const int bg = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (blockIdx.x == 0 && bg == 0)
    for (int i = threadIdx.x; i < a.iters; i += 256) a.flag_cnt[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.offsets[(size_t)bg * (a.C + 1) + a.C] = a.Nc;
  const T* K = static_cast<const T*>(a.k) + (size_t)bg * a.N * kD;
  const T* V = static_cast<const T*>(a.v) + (size_t)bg * a.N * kD;
  T* ks = static_cast<T*>(a.ks) + (size_t)bg * a.NS * kD;
  T* vs = static_cast<T*>(a.vs) + (size_t)bg * a.NS * kD;
  for (int r = blockIdx.x * 4 + w; r < a.NS; r += gridDim.x * 4) {
    // steady row r -> position: the first `sink` positions, then the last `window`
    const int pos = (a.NS == a.N) ? r : (r < a.sink ? r : a.N - a.window + (r - a.sink));
    for (int j = lane; j < kD; j += 64) {
      ks[(size_t)r * kD + j] = K[(size_t)pos * kD + j];
      vs[(size_t)r * kD + j] = V[(size_t)pos * kD + j];
    }
  }
}

// ============================================================================ k_init
// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): output number r of a stream is the mix of
// state0 + (r + 1) * golden gamma.
__device__ __forceinline__ uint64_t splitmix64_nth(uint64_t state0, uint64_t r) {
  uint64_t z = state0 + (r + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Initial state of segment s of (sequence b, KV head g):
// seed XOR (((b << 40) | (g << 20) | s) * 0xD1B54A32D192ED03) mod 2^64.
__device__ __forceinline__ uint64_t segment_state0(uint64_t seed, int b, int g, int s) {
  const uint64_t sid = ((uint64_t)b << 40) | ((uint64_t)g << 20) | (uint64_t)s;
  return seed ^ (sid * 0xD1B54A32D192ED03ull);
}

constexpr int kInitThreads = 512;
// hash slots of the seed search: a power of two, at least twice the clusters of a segment
inline __host__ __device__ int init_hash_slots(int cs) {
  int h = 2;
  while (h < 2 * cs) h <<= 1;
  return h;
}

// The seed rows of one segment's clusters, one cluster per thread.  The partial Fisher-Yates
// shuffle swaps position r with j_r >= r for r = 0, 1, ..., and cluster r takes the row that ends
// at position r.  That row is the one at position j_r just before step r: the row an earlier step
// r' < r moved there (the last with j_r' = j_r; it brought the row then at position r'), else j_r
// itself.  So each cluster follows that chain back through the draws, with no sequential pass
// over the swaps; the draws equal to a position are found through an open-addressing hash table
// of draw indices keyed by their draw (in LDS, at most half full), not by scanning the earlier
// draws.  Then the thread loads its seed row whole, sums its squares in fp64 in ascending
// coordinate order and stores round(x / ||x||) (a zero row for a zero norm).
template <typename T>
__global__ __launch_bounds__(kInitThreads) void k_init(BuildArgs a) {
  extern __shared__ uint32_t init_lds[];      // draws j_r [Cs], hash slots [init_hash_slots(Cs)]
  const int s = a.seg0 + blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int n_s = seg_len_of(a, s);
  const int cs_eff = min(a.Cs, n_s);
  uint32_t* draw = init_lds;
  int* slot = reinterpret_cast<int*>(init_lds + a.Cs);
  const int HS = init_hash_slots(a.Cs), hshift = 32 - __builtin_ctz((unsigned)HS);
  auto hash = [&](uint32_t v) -> int { return hshift >= 32 ? 0 : (int)((v * 0x9E3779B1u) >> hshift); };
  for (int i = threadIdx.x; i < HS; i += kInitThreads) slot[i] = -1;
  const uint64_t st0 = segment_state0(a.seed, b, g, s);
  // the draws do not depend on the shuffle state: j_r = r + (x_r mod (n_s - r))
  for (int r = threadIdx.x; r < cs_eff; r += kInitThreads)
    draw[r] = (uint32_t)r + (uint32_t)(splitmix64_nth(st0, (uint64_t)r) % (uint64_t)(n_s - r));
  __syncthreads();
  for (int r = threadIdx.x; r < cs_eff; r += kInitThreads) {
    int h = hash(draw[r]);
    while (atomicCAS(&slot[h], -1, r) != -1) h = (h + 1) & (HS - 1);
  }
  __syncthreads();
  // the largest draw index x < t with draw x equal to v, or -1 (the probe ends at an empty slot)
  auto last_draw_before = [&](uint32_t v, int t) -> int {
    int best = -1;
    for (int h = hash(v);; h = (h + 1) & (HS - 1)) {
      const int x = slot[h];
      if (x < 0) break;
      if (draw[x] == v && x < t && x > best) best = x;
    }
    return best;
  };
  const T* K = static_cast<const T*>(a.k) + ((size_t)bg * a.N + a.lo + (size_t)s * a.L) * kD;
  T* mh = static_cast<T*>(a.mhat) + ((size_t)bg * a.C + (size_t)s * a.Cs) * kD;
  constexpr int kPer = 16 / (int)sizeof(T);          // elements per 16-byte piece
  constexpr int kPieces = kD / kPer;
  for (int j = threadIdx.x; j < a.Cs; j += kInitThreads) {
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(mh + (size_t)j * kD);
    if (j >= cs_eff) {
#pragma unroll
      for (int i = 0; i < kPieces; ++i) dst[i] = u32x4_t{0u, 0u, 0u, 0u};
      continue;
    }
    int p = (int)draw[j], t = j;
    for (;;) {
      const int q = last_draw_before((uint32_t)p, t);
      if (q < 0) break;
      p = q;
      t = q;
    }
    const u32x4_t* row = reinterpret_cast<const u32x4_t*>(K + (size_t)p * kD);
    u32x4_t r[kPieces];
#pragma unroll
    for (int i = 0; i < kPieces; ++i) r[i] = row[i];
    auto elem = [&](int e) -> double {               // coordinate e of the row
      const u32x4_t& v = r[e / kPer];
      if constexpr (sizeof(T) == 2) {
        const int k = (e % kPer) >> 1;               // the 32-bit word holding it
        const uint32_t w = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
        return (double)__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
      } else {
        const int k = e % kPer;
        return (double)__uint_as_float(k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w);
      }
    };
    double nrm2 = 0.0;
#pragma unroll
    for (int e = 0; e < kD; ++e) {
#pragma clang fp contract(off)
      const double x = elem(e);
      const double sq = x * x;
      nrm2 = nrm2 + sq;
    }
    if (!(nrm2 > 0.0)) {
#pragma unroll
      for (int i = 0; i < kPieces; ++i) dst[i] = u32x4_t{0u, 0u, 0u, 0u};
      continue;
    }
    const double nrm = __builtin_sqrt(nrm2);
    // the row's bits are re-read for the divisions below rather than 128 fp64 values kept live
#pragma unroll
    for (int i = 0; i < kPieces; ++i) asm volatile("" : "+v"(r[i].x), "+v"(r[i].y), "+v"(r[i].z), "+v"(r[i].w));
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (sizeof(T) == 2) {
          const uint32_t lo = St<T>::from_f64(elem(i * kPer + 2 * q) / nrm);
          const uint32_t hi = St<T>::from_f64(elem(i * kPer + 2 * q + 1) / nrm);
          w[q] = lo | (hi << 16);
        } else {
          w[q] = __float_as_uint(St<T>::from_f64(elem(i * kPer + q) / nrm));
        }
      }
      dst[i] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
}

// ============================================================================ k_assign
// Per element type: centroid rows per LDS chunk, LDS row stride (bytes, padded against bank
// conflicts) and waves per block (each wave scores 4 tiles of 16 keys).  bf16 keys fit 128
// VGPRs, so 16 waves (4 per SIMD) share one staged chunk; fp32 keys take twice the registers.
template <typename T> struct AssignCfg;
template <> struct AssignCfg<uint16_t> { static constexpr int kChunk = 512, kStride = 272, kWaves = 16; };
template <> struct AssignCfg<float> { static constexpr int kChunk = 256, kStride = 528, kWaves = 8; };
template <typename T> constexpr int assign_threads() { return 64 * AssignCfg<T>::kWaves; }
constexpr int64_t kAssignBlocksTarget = 256;       // one block per CU
constexpr int kAssignListCap = 2048;   // uncertain keys a resident block re-decides from its LDS list
constexpr int kAssignKeyWaves = 8;     // waves that re-decide one key (one centroid per thread)
template <typename T> constexpr size_t assign_lds_bytes(bool resident) {
  return (size_t)AssignCfg<T>::kChunk * AssignCfg<T>::kStride +
         (resident ? (size_t)kAssignListCap * 4 + (size_t)(AssignCfg<T>::kWaves / kAssignKeyWaves) * kD * 8 : 0);
}

// Running state of one key over the 4-centroid groups seen so far: the largest and second-largest
// group maximum of the fp32 scores, and the group holding the largest.  Every centroid outside
// the best group scores at most b2; the best group's own four scores are recomputed at the end.
struct Best2 {
  float b1, b2;
  int grp;
};

// Fold the group of centroids 4 grp .. 4 grp + 3 (an equal later group does not replace the
// best: lower ids win ties, and b2 then equals b1 so that the key is re-decided exactly).
__device__ __forceinline__ void best2_fold4(Best2& t, float a0, float a1, float a2, float a3, int grp) {
  const float g = fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
  const bool nw = g > t.b1;
  t.b2 = __builtin_amdgcn_fmed3f(t.b1, t.b2, g);            // b1 >= b2: the new second largest
  t.b1 = fmaxf(t.b1, g);
  t.grp = nw ? grp : t.grp;
}

// Merge the state of lane (lane ^ m): the two largest group maxima of the union, the lower group
// on ties.
__device__ __forceinline__ void best2_merge_xor(Best2& t, int m) {
  const float o1 = __shfl_xor(t.b1, m), o2 = __shfl_xor(t.b2, m);
  const int og = __shfl_xor(t.grp, m);
  const bool take = o1 > t.b1 || (o1 == t.b1 && og < t.grp);
  t.b2 = fmaxf(fmaxf(fminf(t.b1, o1), t.b2), o2);
  if (take) { t.b1 = o1; t.grp = og; }
}

// Keys are the MFMA B operand (column = key), held in registers; the segment's centroid
// directions are staged in LDS in chunks and fed as the A operand (row = centroid).  Lane (lr,
// lg) of an output tile holds centroids 4 lg .. 4 lg + 3 of the 16-centroid tile for key lr and
// folds their maximum into the key's running best two group maxima.  At the end the four scores
// of the best group are recomputed, which names the best centroid; the choice is certified when
// it leads every other centroid (the group's other three, and the second-best group maximum) by
// more than twice the fp32 error bound, otherwise the key goes to the fp64 re-decision list.
// With every centroid resident in LDS the block re-decides its own listed keys after its last
// pass (no separate launch: the build's assignment steps took 1.44 + 0.13 ms in two kernels,
// 1.51 ms in one); otherwise k_rescore takes the list.
template <typename T, bool kResident>
__global__ __launch_bounds__(assign_threads<T>()) void k_assign(BuildArgs a, int it) {
  extern __shared__ __attribute__((aligned(16))) unsigned char clds[];
  constexpr int CH = AssignCfg<T>::kChunk, STR = AssignCfg<T>::kStride;
  constexpr int NT = assign_threads<T>();          // 64 keys per wave and pass
  __shared__ int f_cnt;                            // resident: keys on the block's re-decision list
  __shared__ double rd_best[AssignCfg<T>::kWaves];
  __shared__ int rd_id[AssignCfg<T>::kWaves];
  const int s = a.seg0 + blockIdx.y, bg = blockIdx.z;
  const int n_s = seg_len_of(a, s);
  const int cs_eff = min(a.Cs, n_s);
  if ((int)blockIdx.x * NT >= n_s) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;
  const T* K = static_cast<const T*>(a.k) + ((size_t)bg * a.N + a.lo + (size_t)s * a.L) * kD;
  const T* mh = static_cast<const T*>(a.mhat) + ((size_t)bg * a.C + (size_t)s * a.Cs) * kD;
  constexpr bool resident = kResident;            // one staged chunk holds every centroid
  constexpr int Q = kD * (int)sizeof(T) / 16;      // 16-byte pieces per centroid row
  // stage centroid rows [c0, c0 + ch16) into LDS (rows past cs_eff are zero)
  auto stage = [&](int c0, int ch, int ch16) {
    for (int idx = threadIdx.x; idx < ch16 * Q; idx += NT) {
      const int r = idx / Q, q = idx - r * Q;
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (r < ch) val = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const unsigned char*>(mh + (size_t)(c0 + r) * kD) + q * 16);
      *reinterpret_cast<u32x4_t*>(clds + r * STR + q * 16) = val;
    }
  };
  if constexpr (resident) {
    if (threadIdx.x == 0) f_cnt = 0;
    stage(0, cs_eff, (cs_eff + 15) & ~15);
    __syncthreads();
  }

  // The block's passes: keys [p NT, (p + 1) NT) for p = blockIdx.x, blockIdx.x + gridDim.x, ...
  // With every centroid resident there is no barrier between passes, so the waves drift apart
  // and one wave's loads and list updates overlap the others' matrix work.
  for (int key0 = blockIdx.x * NT; key0 < n_s; key0 += gridDim.x * NT) {
  Best2 tk[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) { tk[kt].b1 = -INFINITY; tk[kt].b2 = -INFINITY; tk[kt].grp = 0; }
  // key (lane & 15) of tile kt.  bf16: matrix step st takes dims 32 st + 8 lg .. +8 of keys and
  // centroids, so that one load reads 64 contiguous bytes of each of 16 key rows; fp32: lane
  // group lg holds dims 32 lg .. 32 lg + 31
  constexpr int KE = sizeof(T) == 2 ? 4 : 32;      // bf16: 4 x 8 elements; fp32: 32 elements
  typedef typename std::conditional<sizeof(T) == 2, bf16x8_t, float>::type KElem;
  KElem kb[4][KE];
  // keys past the segment read its last key (in bounds) and are never written back
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int i = min(key0 + w * 64 + kt * 16 + lr, n_s - 1);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < 4; ++st) kb[kt][st] = *reinterpret_cast<const bf16x8_t*>(K + (size_t)i * kD + 32 * st + 8 * lg);
    } else {
#pragma unroll
      for (int st = 0; st < 32; st += 8) {
        float tmp[8];
        St<float>::load8(reinterpret_cast<const float*>(K) + (size_t)i * kD + 32 * lg + st, tmp);
#pragma unroll
        for (int e = 0; e < 8; ++e) kb[kt][st + e] = tmp[e];
      }
    }
  }

  for (int c0 = 0; c0 < cs_eff; c0 += CH) {
    const int ch = min(CH, cs_eff - c0);
    const int ch16 = (ch + 15) & ~15;
    if constexpr (!resident) {
      __syncthreads();
      stage(c0, ch, ch16);
      __syncthreads();
    }
    const int nct = ch16 / 16;
    // one 16-centroid tile: every tile but a ragged last one takes the unmasked path
    auto tile = [&](int ct, bool ragged) {
      const int grp = (c0 + ct * 16) / 4 + lg;
      f32x4_t acc[4];
      if constexpr (sizeof(T) == 2) {
        // one 32-dim slice of the 16 centroid rows at a time, against the four key tiles
        const unsigned char* rp = clds + (ct * 16 + lr) * STR + 16 * lg;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8_t ca = *reinterpret_cast<const bf16x8_t*>(rp + 64 * st);
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca, kb[kt][st], acc[kt], 0, 0, 0);
        }
      } else {
        const float* rp = reinterpret_cast<const float*>(clds + (ct * 16 + lr) * STR) + 32 * lg;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 32; st += 4) {
          const u32x4_t cv = *reinterpret_cast<const u32x4_t*>(rp + st);
          const float cf[4] = {__uint_as_float(cv.x), __uint_as_float(cv.y), __uint_as_float(cv.z), __uint_as_float(cv.w)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
              acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(cf[e], kb[kt][st + e], acc[kt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        float v[4] = {acc[kt][0], acc[kt][1], acc[kt][2], acc[kt][3]};
        if (ragged) {
#pragma unroll
          for (int r = 0; r < 4; ++r) if (4 * grp + r >= cs_eff) v[r] = -INFINITY;
        }
        best2_fold4(tk[kt], v[0], v[1], v[2], v[3], grp);
      }
    };
    const int nfull = (c0 + ch16 <= cs_eff) ? nct : nct - 1;
    for (int ct = 0; ct < nfull; ++ct) tile(ct, false);
    if (nfull < nct) tile(nct - 1, true);
  }

  // combine the four lane groups holding disjoint centroid subsets of the same key
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) { best2_merge_xor(tk[kt], 16); best2_merge_xor(tk[kt], 32); }
  // key norms for the error bound: the diagonal of K K^T for each 16-key tile, on the matrix
  // cores from the key registers (fp32 sums of the exact squares; their relative error, under
  // 128 * 2^-24, is covered by the 2^-10 inflation below).  D[i][i] sits in lane i + 16 (i / 4),
  // component i % 4.
  auto diag_of = [&](const f32x4_t& dd) -> float {
    const float dg = (lr & 3) == 0 ? dd[0] : (lr & 3) == 1 ? dd[1] : (lr & 3) == 2 ? dd[2] : dd[3];
    return __shfl(dg, lr + 16 * (lr >> 2));
  };
  auto knorm_of = [&](int kt) -> float {
    f32x4_t dd = {0.f, 0.f, 0.f, 0.f};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < 4; ++st) dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kt][st], kb[kt][st], dd, 0, 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) dd = __builtin_amdgcn_mfma_f32_16x16x4f32(kb[kt][e], kb[kt][e], dd, 0, 0, 0);
    }
    return sqrtf(diag_of(dd));
  };

  // the winning group's four scores, recomputed (bf16 with resident centroids: on the matrix
  // cores; otherwise on the vector units, each lane its 32 dims, then summed over the four lane
  // groups), name the best centroid; certify it against the best of the rest: the group's other
  // three and the exact second-best fp32 score overall
  int flagged[4];
  // lane's 32-dim part of <key of tile kt, centroid c>; rows from LDS when resident, else global
  auto part_dot = [&](int kt, int c) -> float {
    float acc = 0.f;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4_t cv = *reinterpret_cast<const u32x4_t*>(clds + c * STR + 64 * st + 16 * lg);
        const u32x4_t kw = __builtin_bit_cast(u32x4_t, kb[kt][st]);
        acc = dot2_bf16(cv.x, kw.x, acc);
        acc = dot2_bf16(cv.y, kw.y, acc);
        acc = dot2_bf16(cv.z, kw.z, acc);
        acc = dot2_bf16(cv.w, kw.w, acc);
      }
    } else {
      const float* cr = reinterpret_cast<const float*>(clds + c * STR) + 32 * lg;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc += cr[e] * kb[kt][e];
    }
    return acc;
  };
  auto part_dot_global = [&](int kt, int c) -> float {
    float acc = 0.f;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4_t cv = *reinterpret_cast<const u32x4_t*>(mh + (size_t)c * kD + 32 * st + 8 * lg);
        const u32x4_t kw = __builtin_bit_cast(u32x4_t, kb[kt][st]);
        acc = dot2_bf16(cv.x, kw.x, acc);
        acc = dot2_bf16(cv.y, kw.y, acc);
        acc = dot2_bf16(cv.z, kw.z, acc);
        acc = dot2_bf16(cv.w, kw.w, acc);
      }
    } else {
      const float* cr = reinterpret_cast<const float*>(mh) + (size_t)c * kD + 32 * lg;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc += cr[e] * kb[kt][e];
    }
    return acc;
  };
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int grp = tk[kt].grp;
    float p[4];
    if constexpr (resident && sizeof(T) == 2) {
      // on the matrix cores: A row i = centroid 4 grp_i + r of key i (each lane gathers its own
      // key's row from LDS), B = the key tile; the wanted scores are the diagonal of each product
      // (after the merges every lane of key lr holds its group)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const unsigned char* rp = clds + min(4 * grp + r, cs_eff - 1) * STR + 16 * lg;
        f32x4_t dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st)
          dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(rp + 64 * st), kb[kt][st], dd, 0, 0, 0);
        p[r] = 4 * grp + r < cs_eff ? diag_of(dd) : -INFINITY;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = min(4 * grp + r, cs_eff - 1);
        float acc;
        if constexpr (resident) acc = part_dot(kt, c);
        else acc = part_dot_global(kt, c);
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        p[r] = 4 * grp + r < cs_eff ? acc : -INFINITY;
      }
    }
    int rb = 0;
#pragma unroll
    for (int r = 1; r < 4; ++r) if (p[r] > p[rb]) rb = r;
    float b2 = tk[kt].b2;
#pragma unroll
    for (int r = 0; r < 4; ++r) if (r != rb) b2 = fmaxf(b2, p[r]);
    const float kn_kt = knorm_of(kt);
    const int i = key0 + w * 64 + kt * 16 + lr;
    flagged[kt] = 0;
    if (lg == 0 && i < n_s) {
      const size_t gi = (size_t)bg * a.Nc + (size_t)s * a.L + i;
      const double kn = (double)kn_kt * (1.0 + 1.0 / 1024);
      const double delta = 2.0 * (kD + 2) * 5.9604644775390625e-08 * kn * 1.01 + 1e-30;
      a.assign[gi] = 4 * grp + rb;
      flagged[kt] = !((double)p[rb] - (double)b2 > 2.0 * delta);
    }
  }
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const uint64_t m = __ballot(flagged[kt]);
    if (m == 0) continue;
    uint32_t base = 0;
    if (lane == 0) base = resident ? (uint32_t)atomicAdd(&f_cnt, __popcll(m)) : atomicAdd(&a.flag_cnt[it], (uint32_t)__popcll(m));
    base = __builtin_amdgcn_readlane(base, 0);
    if (flagged[kt]) {
      const uint32_t pos = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
      const int i = key0 + w * 64 + kt * 16 + lr;
      const size_t gi = (size_t)bg * a.Nc + (size_t)s * a.L + i;
      if constexpr (resident) {
        // the block's list in LDS; past its capacity the key is marked in place (-1)
        if (pos < (uint32_t)kAssignListCap) reinterpret_cast<int*>(clds + CH * STR)[pos] = i;
        else a.assign[gi] = -1;
      } else {
        a.flag_list[pos] = (int32_t)gi;
      }
    }
  }
  }  // passes

  if constexpr (resident) {
    // The fp64 re-decision of the block's uncertain keys, against the centroids still in LDS:
    // kAssignKeyWaves waves per key, one centroid per thread, the canonical score (exact products
    // added in ascending coordinate order in fp64: a fused multiply-add of an exact product rounds
    // as the addition does), the block argmax with ties to the lower id.
    // Keys past the list's capacity were marked in place; the block then finds them by reading
    // back its own keys' assignments, one pass of keys at a time.
    int* flist = reinterpret_cast<int*>(clds + CH * STR);
    double* fkey = reinterpret_cast<double*>(clds + CH * STR + kAssignListCap * 4);
    constexpr int KPR = AssignCfg<T>::kWaves / kAssignKeyWaves;     // keys per round
    const int kg = w / kAssignKeyWaves, gt = threadIdx.x - kg * kAssignKeyWaves * 64;
    auto redecide = [&](int n_list) {
      for (int r0 = 0; r0 < n_list; r0 += KPR) {
        const int e = r0 + kg;
        const int i = e < n_list ? flist[e] : -1;
        if (i >= 0 && gt < kD) fkey[kg * kD + gt] = (double)St<T>::f(K[(size_t)i * kD + gt]);
        __syncthreads();
        double best = -INFINITY;
        int bj = 0x7fffffff;
        if (i >= 0 && gt < cs_eff) {
#pragma clang fp contract(off)
          const double* kq = fkey + kg * kD;
          const unsigned char* crow = clds + gt * STR;
          double acc = 0.0;
          if constexpr (sizeof(T) == 2) {
#pragma unroll 4
            for (int q = 0; q < kD / 8; ++q) {
              const u32x4_t cv = *reinterpret_cast<const u32x4_t*>(crow + 16 * q);
              const uint32_t wd[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                acc = __builtin_fma(kq[8 * q + 2 * h], (double)__uint_as_float(wd[h] << 16), acc);
                acc = __builtin_fma(kq[8 * q + 2 * h + 1], (double)__uint_as_float(wd[h] & 0xffff0000u), acc);
              }
            }
          } else {
#pragma unroll 4
            for (int q = 0; q < kD / 4; ++q) {
              const u32x4_t cv = *reinterpret_cast<const u32x4_t*>(crow + 16 * q);
              const uint32_t wd[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
              for (int h = 0; h < 4; ++h) acc = __builtin_fma(kq[4 * q + h], (double)__uint_as_float(wd[h]), acc);
            }
          }
          best = acc;
          bj = gt;
        }
#pragma unroll
        for (int m = 32; m > 0; m >>= 1) {
          const double ob = __shfl_xor(best, m);
          const int oj = __shfl_xor(bj, m);
          if (ob > best || (ob == best && oj < bj)) { best = ob; bj = oj; }
        }
        if (lane == 0) { rd_best[w] = best; rd_id[w] = bj; }
        __syncthreads();
        if (gt == 0 && i >= 0) {
          for (int x = 1; x < kAssignKeyWaves; ++x) {
            const double ob = rd_best[w + x];
            const int oj = rd_id[w + x];
            if (ob > best || (ob == best && oj < bj)) { best = ob; bj = oj; }
          }
          a.assign[(size_t)bg * a.Nc + (size_t)s * a.L + i] = bj;
        }
        __syncthreads();                       // fkey and the partials are reused next round
      }
    };
    __syncthreads();
    const int n_flag = f_cnt;
    redecide(min(n_flag, kAssignListCap));
    if (n_flag > kAssignListCap) {
      for (int key0 = blockIdx.x * NT; key0 < n_s; key0 += gridDim.x * NT) {
        if (threadIdx.x == 0) f_cnt = 0;
        __syncthreads();
        const int i = key0 + (int)threadIdx.x;
        if (i < n_s && a.assign[(size_t)bg * a.Nc + (size_t)s * a.L + i] < 0) flist[atomicAdd(&f_cnt, 1)] = i;
        __syncthreads();
        redecide(f_cnt);
      }
    }
  }
}

// ============================================================================ k_rescore
// The keys the assignment could not certify when the centroids did not fit in LDS, one per
// workgroup at a time: each thread forms the
// canonical scores of its centroids (c = t, t + 512, ...) with the 128 exact products added in
// ascending coordinate order, and a block argmax (ties to the lower id) names the cluster.  The
// dependent memory round trips are few: the list count and the workgroup's first entry are read
// together, then the key row (staged in LDS in fp64) and the first centroid row of every thread
// are requested together.
constexpr int kRescoreThreads = 512;

template <typename T>
__global__ __launch_bounds__(kRescoreThreads) void k_rescore(BuildArgs a, int it) {
#pragma clang fp contract(off)
  constexpr int NW = kRescoreThreads / 64;
  constexpr int kPer = 16 / (int)sizeof(T);            // elements per 16-byte piece
  constexpr int kBatches = kD / (16 * kPer);            // 16-piece batches per row: 1 (bf16), 2 (fp32)
  __shared__ double kx[kD];
  __shared__ double rb[NW];
  __shared__ int rj[NW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t cap = (uint32_t)a.BG * (uint32_t)a.Nc;  // list slots (one per clustered token)
  uint32_t e = blockIdx.x;
  const uint32_t n = a.flag_cnt[it];
  int packed = a.flag_list[min(e, cap - 1u)];           // read beside the count; used only if e < n
  while (e < n) {
    const int bg = packed / a.Nc, ci = packed - bg * a.Nc;
    const int s = ci / a.L;
    const int cs_eff = min(a.Cs, seg_len_of(a, s));
    const T* krow = static_cast<const T*>(a.k) + ((size_t)bg * a.N + a.lo + ci) * kD;
    const T* mh = static_cast<const T*>(a.mhat) + ((size_t)bg * a.C + (size_t)s * a.Cs) * kD;
    // the key's 16-byte pieces (threads < kD / kPer) and the first batch of this thread's first
    // centroid row (clamped into the segment's rows; unused past cs_eff) go out together
    u32x4_t kpc = {0u, 0u, 0u, 0u};
    if (tid < kD / kPer) kpc = reinterpret_cast<const u32x4_t*>(krow)[tid];
    u32x4_t r[16];
    {
      const u32x4_t* crow = reinterpret_cast<const u32x4_t*>(mh + (size_t)min(tid, cs_eff - 1) * kD);
#pragma unroll
      for (int i = 0; i < 16; ++i) r[i] = crow[i];
    }
    if (tid < kD / kPer) {
      const uint32_t wd[4] = {kpc.x, kpc.y, kpc.z, kpc.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (sizeof(T) == 2) {
          kx[tid * kPer + 2 * q] = (double)__uint_as_float(wd[q] << 16);
          kx[tid * kPer + 2 * q + 1] = (double)__uint_as_float(wd[q] & 0xffff0000u);
        } else {
          kx[tid * kPer + q] = (double)__uint_as_float(wd[q]);
        }
      }
    }
    __syncthreads();
    double best = -INFINITY;
    int bj = 0x7fffffff;
    for (int j = tid; j < cs_eff; j += kRescoreThreads) {
      const u32x4_t* crow = reinterpret_cast<const u32x4_t*>(mh + (size_t)j * kD);
      const double* kq = kx + opaque_zero();          // the key's values re-read per centroid
      double acc = 0.0;
#pragma unroll
      for (int h = 0; h < kBatches; ++h) {
        if (j != tid || h > 0) {
#pragma unroll
          for (int i = 0; i < 16; ++i) r[i] = crow[h * 16 + i];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t wd[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d0 = (h * 16 + i) * kPer;
            if constexpr (sizeof(T) == 2) {
              const double p0 = kq[d0 + 2 * q] * (double)__uint_as_float(wd[q] << 16);
              acc = acc + p0;
              const double p1 = kq[d0 + 2 * q + 1] * (double)__uint_as_float(wd[q] & 0xffff0000u);
              acc = acc + p1;
            } else {
              const double p = kq[d0 + q] * (double)__uint_as_float(wd[q]);
              acc = acc + p;
            }
          }
        }
      }
      if (acc > best || bj == 0x7fffffff) { best = acc; bj = j; }
    }
    // block argmax, ties to the lower id
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
      const double ob = __shfl_xor(best, m);
      const int oj = __shfl_xor(bj, m);
      if (ob > best || (ob == best && oj < bj)) { best = ob; bj = oj; }
    }
    if (lane == 0) { rb[w] = best; rj[w] = bj; }
    __syncthreads();
    if (tid == 0) {
      for (int i = 1; i < NW; ++i)
        if (rb[i] > best || (rb[i] == best && rj[i] < bj)) { best = rb[i]; bj = rj[i]; }
      a.assign[(size_t)bg * a.Nc + ci] = bj;
    }
    e += gridDim.x;
    if (e < n) packed = a.flag_list[e];
    __syncthreads();
  }
}

// ============================================================================ k_csr
// One workgroup per segment, whose tokens are split into 16 contiguous ranges of whole 64-token
// steps, one per wave.  (1) Each wave counts its range's ids into its own row of a [16][Cs] table
// of 16-bit counts; (2) the thread owning cluster c turns column c into exclusive prefixes over
// the waves (the tokens of id c in earlier ranges) and the total; (3) a block scan of the totals
// gives the offsets; (4) each wave walks its range in order, 64 tokens a step: a token's slot is
// its id's offset, plus the id's tokens before this step (its entry in the wave's table row,
// which every lane then advances with an LDS atomic, so that the entry read back gives the id's
// count in the step), plus its rank among the equal ids of the step (0 for an id that occurs
// once; one ballot for each id that occurs more than once).
// Only (1)-(3) need block barriers.  Counts fit 16 bits: a segment holds at most 65536 tokens,
// and a prefix before a wave's range at most 15/16 of them.
constexpr int kCsrThreads = 1024;
constexpr int kCsrWaves = kCsrThreads / 64;
constexpr int kCsrRegSteps = 8;     // steps of ids a lane keeps in registers from (1) to (4)
inline size_t csr_lds_bytes(int Cs) {
  const size_t cs2 = (size_t)((Cs + 1) & ~1);
  return (size_t)kCsrWaves * cs2 * 2 + (size_t)Cs * 4;
}

__global__ __launch_bounds__(kCsrThreads) void k_csr(BuildArgs a) {
  extern __shared__ uint32_t csr_lds[];   // tbl[16][Cs2] (u16), loc[Cs]
  __shared__ int iscr[32];
  const int s = a.seg0 + blockIdx.x, bg = blockIdx.y;
  const int n_s = seg_len_of(a, s);
  const int Cs = a.Cs, Cs2 = (Cs + 1) & ~1;
  uint16_t* tbl = reinterpret_cast<uint16_t*>(csr_lds);
  uint32_t* loc = csr_lds + kCsrWaves * Cs2 / 2;
  const int32_t* asg = a.assign + (size_t)bg * a.Nc + (size_t)s * a.L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int R = (n_s + 64 * kCsrWaves - 1) / (64 * kCsrWaves) * 64;   // tokens per wave
  const int t0 = min(n_s, w * R), t1 = min(n_s, t0 + R);

  for (int x = tid; x < kCsrWaves * Cs2 / 2; x += kCsrThreads) csr_lds[x] = 0u;
  int kr[kCsrRegSteps];
#pragma unroll
  for (int u = 0; u < kCsrRegSteps; ++u) {
    const int i = t0 + 64 * u + lane;
    kr[u] = i < t1 ? asg[i] : -1;
  }
  __syncthreads();
  // (1) the wave's counts; two 16-bit counts share a word, added to with 32-bit atomics
  auto count = [&](int key) {
    if (key >= 0) atomicAdd(&csr_lds[(w * Cs2 + key) >> 1], 1u << (16 * (key & 1)));
  };
#pragma unroll
  for (int u = 0; u < kCsrRegSteps; ++u) count(kr[u]);
  for (int i = t0 + 64 * kCsrRegSteps + lane; i < t1; i += 64) count(asg[i]);
  __syncthreads();
  // (2) prefixes over the waves, totals (kept in loc until the scan)
  const int per = (Cs + kCsrThreads - 1) / kCsrThreads;
  const int j0 = min(Cs, tid * per), j1 = min(Cs, j0 + per);
  int my = 0;
  for (int j = j0; j < j1; ++j) {
    int run = 0;
    for (int ww = 0; ww < kCsrWaves; ++ww) {
      const int x = tbl[ww * Cs2 + j];
      tbl[ww * Cs2 + j] = (uint16_t)run;
      run += x;
    }
    loc[j] = (uint32_t)run;
    my += run;
  }
  // (3) offsets
  int tot;
  int ex = block_exclusive_scan<kCsrThreads>(my, iscr, &tot);
  const int cbase = s * Cs;
  for (int j = j0; j < j1; ++j) {
    const int c = (int)loc[j];
    a.sizes[(size_t)bg * a.C + cbase + j] = (int32_t)c;
    a.offsets[(size_t)bg * (a.C + 1) + cbase + j] = s * a.L + ex;
    loc[j] = (uint32_t)ex;
    ex += c;
  }
  __syncthreads();
  // (4) the wave's range in order
  int32_t* perm = a.perm + (size_t)bg * a.Nc + (size_t)s * a.L;
  const int pos0 = a.lo + s * a.L;
  uint16_t* mine = tbl + w * Cs2;
  auto step = [&](int i, int key) {
    const bool v = key >= 0;
    const int before = v ? (int)mine[key] : 0;
    wave_lds_sync();                  // every lane has read its id's count before any is added to
    if (v) atomicAdd(&csr_lds[(w * Cs2 + key) >> 1], 1u << (16 * (key & 1)));
    wave_lds_sync();
    // the step's tokens of this id (16-bit difference: the count reaches 65536 only at the last
    // step of a segment that is one cluster), and the rank among them in lane order, found by one
    // ballot per id that occurs more than once
    const int cnt = v ? (int)(uint16_t)(mine[key] - (uint16_t)before) : 0;
    int rank = 0;
    uint64_t dup = __ballot(cnt > 1);
    while (dup != 0ull) {
      const int l = __ffsll((unsigned long long)dup) - 1;
      const int k = __builtin_amdgcn_readlane(key, l);
      const uint64_t m = __ballot(key == k);
      if (key == k) rank = __popcll(m & ((1ull << lane) - 1ull));
      dup &= ~m;
    }
    if (v) perm[(int)loc[key] + before + rank] = pos0 + i;
  };
#pragma unroll
  for (int u = 0; u < kCsrRegSteps; ++u)
    if (t0 + 64 * u < t1) step(t0 + 64 * u + lane, kr[u]);
  for (int b0 = t0 + 64 * kCsrRegSteps; b0 < t1; b0 += 64) {
    const int i = b0 + lane;
    step(i, i < t1 ? asg[i] : -1);
  }
}

// ============================================================================ k_final / k_update2
// Final (last iteration): one wave per cluster; lane owns dims 2*lane, 2*lane+1.  Members are
// summed in fp64 in ascending position (the CSR order), 16 rows fetched ahead of the sums, the
// positions of 64 members in one load; mean key, value sum and the cluster-major K/V copies.
template <typename T>
__global__ __launch_bounds__(512) void k_final(BuildArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int s = a.seg0 + blockIdx.y, bg = blockIdx.z;
  const int j = blockIdx.x * 8 + w;
  if (j >= a.Cs) return;
  const int n_s = seg_len_of(a, s);
  const int cs_eff = min(a.Cs, n_s);
  const int c = s * a.Cs + j;
  const size_t cidx = (size_t)bg * a.C + c;
  T* dst = static_cast<T*>(a.mu) + cidx * kD;
  T* sv = static_cast<T*>(a.sv) + cidx * kD;
  const int n = j < cs_eff ? a.sizes[cidx] : 0;
  const int start = j < cs_eff ? a.offsets[(size_t)bg * (a.C + 1) + c] : 0;
  const int32_t* perm = a.perm + (size_t)bg * a.Nc;
  const T* K = static_cast<const T*>(a.k) + (size_t)bg * a.N * kD;
  const T* V = static_cast<const T*>(a.v) + (size_t)bg * a.N * kD;
  T* kp = static_cast<T*>(a.kp) + (size_t)bg * a.Nc * kD;
  T* vp = static_cast<T*>(a.vp) + (size_t)bg * a.Nc * kD;
  double k0 = 0.0, k1 = 0.0, v0 = 0.0, v1 = 0.0;
  int p = 0;                          // member positions, 64 at a time (one per lane)
  for (int m0 = 0; m0 < n; m0 += 16) {
    const int cnt = min(16, n - m0);
    if ((m0 & 63) == 0 && m0 + lane < n) p = perm[start + m0 + lane];
    T kx[16][2], vx[16][2];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int pos = __shfl(p, (m0 & 63) + u);
      if (u < cnt) {
        kx[u][0] = K[(size_t)pos * kD + 2 * lane];
        kx[u][1] = K[(size_t)pos * kD + 2 * lane + 1];
        vx[u][0] = V[(size_t)pos * kD + 2 * lane];
        vx[u][1] = V[(size_t)pos * kD + 2 * lane + 1];
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u < cnt) {
#pragma clang fp contract(off)
        k0 = k0 + (double)St<T>::f(kx[u][0]);
        k1 = k1 + (double)St<T>::f(kx[u][1]);
        v0 = v0 + (double)St<T>::f(vx[u][0]);
        v1 = v1 + (double)St<T>::f(vx[u][1]);
        const size_t r = (size_t)(start + m0 + u) * kD;
        kp[r + 2 * lane] = kx[u][0]; kp[r + 2 * lane + 1] = kx[u][1];
        vp[r + 2 * lane] = vx[u][0]; vp[r + 2 * lane + 1] = vx[u][1];
      }
    }
  }
  if (n > 0) {
    const double dn = (double)n;
    dst[2 * lane] = St<T>::from_f64(k0 / dn);
    dst[2 * lane + 1] = St<T>::from_f64(k1 / dn);
    sv[2 * lane] = St<T>::from_f64(v0);
    sv[2 * lane + 1] = St<T>::from_f64(v1);
  } else {                            // empty, or past the segment's clusters: zero
    dst[2 * lane] = St<T>::from_f64(0.0); dst[2 * lane + 1] = St<T>::from_f64(0.0);
    sv[2 * lane] = St<T>::from_f64(0.0); sv[2 * lane + 1] = St<T>::from_f64(0.0);
  }
}

// Update (every iteration but the last): two clusters per wave, whose loads are issued together
// (sizes and offsets, then member positions, then member rows), so that each wave keeps twice
// the round trips in flight; the two norms are then summed by lanes 0 and 1 at once.  Members are
// summed in fp64 in ascending position (the CSR order), as in k_final (one wave per cluster:
// update 63.9 -> 53.9 us per launch).
constexpr int kUpdateWaves = 4;
template <typename T>
__global__ __launch_bounds__(64 * kUpdateWaves) void k_update2(BuildArgs a) {
  __shared__ double buf[kUpdateWaves][2][kD];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int s = a.seg0 + blockIdx.y, bg = blockIdx.z;
  const int j0 = (blockIdx.x * kUpdateWaves + w) * 2;
  const int n_s = seg_len_of(a, s);
  const int cs_eff = min(a.Cs, n_s);
  if (j0 >= cs_eff) return;                 // clusters past cs_eff keep their direction
  const int32_t* perm = a.perm + (size_t)bg * a.Nc;
  const T* K = static_cast<const T*>(a.k) + (size_t)bg * a.N * kD;
  int n[2], start[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = j0 + q, c = s * a.Cs + j;
    const bool ok = j < cs_eff;
    n[q] = ok ? a.sizes[(size_t)bg * a.C + c] : 0;
    start[q] = ok ? a.offsets[(size_t)bg * (a.C + 1) + c] : 0;
  }
  const int nmax = max(n[0], n[1]);
  double x[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  int p[2] = {0, 0};                        // member positions, 64 at a time (one per lane)
  for (int m0 = 0; m0 < nmax; m0 += 16) {
    if ((m0 & 63) == 0) {
#pragma unroll
      for (int q = 0; q < 2; ++q) if (m0 + lane < n[q]) p[q] = perm[start[q] + m0 + lane];
    }
    // the lane's two elements of a member row as one 4-byte (bf16) or 8-byte (fp32) load
    using Pair = typename std::conditional<sizeof(T) == 2, uint32_t, uint2>::type;
    Pair kx[2][16];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int pos = __shfl(p[q], (m0 & 63) + u);
        if (m0 + u < n[q]) kx[q][u] = *reinterpret_cast<const Pair*>(K + (size_t)pos * kD + 2 * lane);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (m0 + u < n[q]) {
#pragma clang fp contract(off)
          float e0, e1;
          if constexpr (sizeof(T) == 2) {
            e0 = __uint_as_float(kx[q][u] << 16);
            e1 = __uint_as_float(kx[q][u] & 0xffff0000u);
          } else {
            e0 = __uint_as_float(kx[q][u].x);
            e1 = __uint_as_float(kx[q][u].y);
          }
          x[q][0] = x[q][0] + (double)e0;
          x[q][1] = x[q][1] + (double)e1;
        }
      }
    }
  }
  // dst = round_dtype(x / ||x||), ||x||^2 summed in fp64 in ascending coordinate order (cluster
  // q's by lane q); a zero sum leaves the direction unchanged
#pragma unroll
  for (int q = 0; q < 2; ++q) { buf[w][q][2 * lane] = x[q][0]; buf[w][q][2 * lane + 1] = x[q][1]; }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double nrm2 = 0.0;
  if (lane < 2) {
#pragma clang fp contract(off)
    const double* row = buf[w][lane];
    for (int d = 0; d < kD; ++d) {
      const double sq = row[d] * row[d];
      nrm2 = nrm2 + sq;
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const double nq = __shfl(nrm2, q);
    if (j0 + q < cs_eff && n[q] > 0 && nq > 0.0) {
      const double nrm = __builtin_sqrt(nq);
      T* dst = static_cast<T*>(a.mhat) + ((size_t)bg * a.C + (size_t)s * a.Cs + j0 + q) * kD;
      dst[2 * lane] = St<T>::from_f64(x[q][0] / nrm);
      dst[2 * lane + 1] = St<T>::from_f64(x[q][1] / nrm);
    }
  }
}

// ============================================================================ launcher
template <typename T>
static hipError_t launch_build_t(const BuildArgs& a, hipStream_t st) {
  const int BG = a.BG;
  {
    const int gx = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(a.NS, 4), 4096));
    prof_begin(WI_STAGE_PREP, st);
    hipLaunchKernelGGL(k_prep<T>, dim3(gx, BG), dim3(256), 0, st, a);
    prof_end(WI_STAGE_PREP, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.Nc == 0 || a.seg0 >= a.nseg) return hipSuccess;
  const int nseg_b = a.nseg - a.seg0;        // segments built by this call
  {
    const size_t lds = (size_t)a.Cs * 4 + (size_t)init_hash_slots(a.Cs) * 4;
    prof_begin(WI_STAGE_INIT, st);
    hipLaunchKernelGGL(k_init<T>, dim3(nseg_b, BG), dim3(kInitThreads), lds, st, a);
    prof_end(WI_STAGE_INIT, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool resident = a.Cs <= AssignCfg<T>::kChunk;   // every centroid of a segment fits in LDS
  const size_t alds = assign_lds_bytes<T>(resident);
  const size_t clds = csr_lds_bytes(a.Cs);
  // assignment blocks per segment: about one block per CU in all (each stages the segment's
  // centroids once and loops over 64-key-per-wave passes), at least one pass each
  const unsigned assign_px = (unsigned)std::max<int64_t>(1, std::min<int64_t>(
      ceil_div(a.L, assign_threads<T>()), ceil_div(kAssignBlocksTarget, (int64_t)nseg_b * BG)));
  for (int it = 0; it < a.iters; ++it) {
    prof_begin(WI_STAGE_ASSIGN, st);
    if (resident)
      hipLaunchKernelGGL((k_assign<T, true>), dim3(assign_px, nseg_b, BG), dim3(assign_threads<T>()),
                         alds, st, a, it);
    else
      hipLaunchKernelGGL((k_assign<T, false>), dim3(assign_px, nseg_b, BG), dim3(assign_threads<T>()),
                         alds, st, a, it);
    prof_end(WI_STAGE_ASSIGN, st);
    if (!resident) {    // a resident assignment re-decides its uncertain keys itself
      prof_begin(WI_STAGE_RESCORE, st);
      hipLaunchKernelGGL(k_rescore<T>, dim3(2048), dim3(kRescoreThreads), 0, st, a, it);
      prof_end(WI_STAGE_RESCORE, st);
    }
    prof_begin(WI_STAGE_CSR, st);
    hipLaunchKernelGGL(k_csr, dim3(nseg_b, BG), dim3(kCsrThreads), clds, st, a);
    prof_end(WI_STAGE_CSR, st);
    if (it + 1 < a.iters) {
      prof_begin(WI_STAGE_UPDATE, st);
      hipLaunchKernelGGL((k_update2<T>), dim3((unsigned)ceil_div(a.Cs, 2 * kUpdateWaves), nseg_b, BG),
                         dim3(64 * kUpdateWaves), 0, st, a);
      prof_end(WI_STAGE_UPDATE, st);
    } else {
      prof_begin(WI_STAGE_FINAL, st);
      hipLaunchKernelGGL((k_final<T>), dim3((unsigned)ceil_div(a.Cs, 8), nseg_b, BG), dim3(512), 0, st, a);
      prof_end(WI_STAGE_FINAL, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static void set_lds_limits() {
  static bool done = false;
  if (done) return;
  const int big = 160 * 1024 - 8192;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_init<float>), hipFuncAttributeMaxDynamicSharedMemorySize, big);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_init<uint16_t>), hipFuncAttributeMaxDynamicSharedMemorySize, big);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_assign<float, true>), hipFuncAttributeMaxDynamicSharedMemorySize, big);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_assign<float, false>), hipFuncAttributeMaxDynamicSharedMemorySize, big);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_assign<uint16_t, true>), hipFuncAttributeMaxDynamicSharedMemorySize, big);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_assign<uint16_t, false>), hipFuncAttributeMaxDynamicSharedMemorySize, big);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_csr), hipFuncAttributeMaxDynamicSharedMemorySize, big);
  done = true;
}

// ============================================================================ k_copy_prefix
// dst[g][0 .. bytes) = src[g][0 .. bytes) for g < G, rows of the source and destination `pitch`
// bytes apart: the leading rows of every (b, KV head) block of an index buffer.  Words of 16 bytes
// when every address and pitch allows, else 4.
template <typename W>
__global__ __launch_bounds__(256) void k_copy_prefix(const unsigned char* src, unsigned char* dst,
                                                     size_t src_pitch, size_t dst_pitch, size_t bytes) {
  const W* s = reinterpret_cast<const W*>(src + (size_t)blockIdx.y * src_pitch);
  W* d = reinterpret_cast<W*>(dst + (size_t)blockIdx.y * dst_pitch);
  const size_t n = bytes / sizeof(W);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) d[i] = s[i];
}

static hipError_t copy_prefix(const void* src, void* dst, size_t src_pitch, size_t dst_pitch, size_t bytes,
                              int G, hipStream_t st) {
  if (bytes == 0 || G == 0) return hipSuccess;
  const bool wide = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | src_pitch |
                      dst_pitch | bytes) & 15) == 0;
  const size_t words = bytes / (wide ? 16 : 4);
  const unsigned gx = (unsigned)std::max<size_t>(1, std::min<size_t>(ceil_div((int64_t)words, 256 * 4), 1024));
  if (wide)
    hipLaunchKernelGGL(k_copy_prefix<u32x4_t>, dim3(gx, G), dim3(256), 0, st,
                       static_cast<const unsigned char*>(src), static_cast<unsigned char*>(dst), src_pitch, dst_pitch, bytes);
  else
    hipLaunchKernelGGL(k_copy_prefix<uint32_t>, dim3(gx, G), dim3(256), 0, st,
                       static_cast<const unsigned char*>(src), static_cast<unsigned char*>(dst), src_pitch, dst_pitch, bytes);
  return hipGetLastError();
}

hipError_t launch_build(const wi_build_params& p, const BuildLayout& L, const void* k, const void* v,
                        const wi_index_view& out, void* ws, hipStream_t st, const wi_index_view* prev,
                        int seg0) {
  set_lds_limits();
  BuildArgs a;
  a.k = k; a.v = v;
  a.mu = out.centroids; a.sv = out.value_sums;
  a.sizes = out.sizes; a.offsets = out.offsets; a.perm = out.perm;
  a.kp = out.k_perm; a.vp = out.v_perm; a.ks = out.k_steady; a.vs = out.v_steady;
  char* base = static_cast<char*>(ws);
  a.mhat = base + L.off_mhat;
  a.assign = reinterpret_cast<int32_t*>(base + L.off_assign);
  a.flag_cnt = reinterpret_cast<uint32_t*>(base + L.off_flag_cnt);
  a.flag_list = reinterpret_cast<int32_t*>(base + L.off_flag_list);
  a.Hkv = p.Hkv; a.N = p.N; a.sink = p.sink; a.window = p.window;
  a.NS = (int)L.NS; a.Nc = (int)L.Nc; a.lo = (L.Nc > 0) ? p.sink : p.N;
  a.L = (int)L.L; a.nseg = (int)L.nseg; a.Cs = p.clusters_per_seg; a.C = (int)L.C;
  a.BG = p.B * p.Hkv; a.iters = p.iters; a.seed = p.seed;
  a.seg0 = seg0;
  if (prev && seg0 > 0) {
    // segments [0, seg0) of every (b, KV head) come from the previous index, whose C and Nc are
    // those of its seg0 segments (the rows of a segment sit at the same places in both)
    const size_t e = p.dtype == WI_BF16 ? 2 : 4;
    const size_t C0 = (size_t)seg0 * p.clusters_per_seg, N0 = (size_t)seg0 * L.L;
    const size_t C1 = (size_t)L.C, N1 = (size_t)L.Nc, d = kD;
    const int G = a.BG;
    hipError_t r;
    if ((r = copy_prefix(prev->centroids, out.centroids, C0 * d * e, C1 * d * e, C0 * d * e, G, st)) != hipSuccess) return r;
    if ((r = copy_prefix(prev->value_sums, out.value_sums, C0 * d * e, C1 * d * e, C0 * d * e, G, st)) != hipSuccess) return r;
    if ((r = copy_prefix(prev->sizes, out.sizes, C0 * 4, C1 * 4, C0 * 4, G, st)) != hipSuccess) return r;
    if ((r = copy_prefix(prev->offsets, out.offsets, (C0 + 1) * 4, (C1 + 1) * 4, C0 * 4, G, st)) != hipSuccess) return r;
    if ((r = copy_prefix(prev->perm, out.perm, N0 * 4, N1 * 4, N0 * 4, G, st)) != hipSuccess) return r;
    if ((r = copy_prefix(prev->k_perm, out.k_perm, N0 * d * e, N1 * d * e, N0 * d * e, G, st)) != hipSuccess) return r;
    if ((r = copy_prefix(prev->v_perm, out.v_perm, N0 * d * e, N1 * d * e, N0 * d * e, G, st)) != hipSuccess) return r;
  }
  return p.dtype == WI_BF16 ? launch_build_t<uint16_t>(a, st) : launch_build_t<float>(a, st);
}

}  // namespace wi
