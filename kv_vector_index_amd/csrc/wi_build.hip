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
//   k_prep      steady-zone copies, fp32 key norms for the error band, counter reset
//   k_init      per segment: SplitMix64-driven partial Fisher-Yates picks the seed rows;
//               directions = rounded unit seed keys
//   then `iters` times:
//     k_assign  MFMA keys x centroid directions (centroids staged in LDS, keys in registers)
//               with a fused running top-2 per key; uncertain keys go to a list
//     k_rescore fp64 canonical argmax for the listed keys
//     k_csr     per segment: counts, offsets and a stable counting scatter -> sizes/offsets/perm
//     k_update  (all but the last iteration) fp64 member sums -> new unit directions
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

// dst = round_dtype(x / ||x||) for a row held as two fp64 values per lane (dims 2*lane, 2*lane+1)
// of one wave.  ||x||^2 is summed in fp64 in ascending coordinate order.  If ||x|| = 0 the row
// is left unchanged (keep = true) or zeroed.  `buf` holds kD doubles of LDS for this wave.
template <typename T>
__device__ void store_unit_direction(double x0, double x1, T* dst, double* buf, bool keep) {
  const int lane = threadIdx.x & 63;
  buf[2 * lane] = x0;
  buf[2 * lane + 1] = x1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double nrm2 = 0.0;
  if (lane == 0) {
#pragma clang fp contract(off)
    for (int j = 0; j < kD; ++j) {
      const double sq = buf[j] * buf[j];
      nrm2 = nrm2 + sq;
    }
  }
  nrm2 = __shfl(nrm2, 0);
  if (nrm2 > 0.0) {
    const double nrm = __builtin_sqrt(nrm2);
    dst[2 * lane] = St<T>::from_f64(x0 / nrm);
    dst[2 * lane + 1] = St<T>::from_f64(x1 / nrm);
  } else if (!keep) {
    dst[2 * lane] = St<T>::from_f64(0.0);
    dst[2 * lane + 1] = St<T>::from_f64(0.0);
  }
  __builtin_amdgcn_wave_barrier();
}

constexpr int kInitThreads = 512;

template <typename T>
__global__ __launch_bounds__(kInitThreads) void k_init(BuildArgs a) {
  extern __shared__ uint32_t init_lds[];      // draws j_r [Cs], then the row array [n_s] (u16)
  __shared__ double buf[kInitThreads / 64][kD];
  const int s = a.seg0 + blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int n_s = seg_len_of(a, s);
  const int cs_eff = min(a.Cs, n_s);
  uint32_t* draw = init_lds;
  uint16_t* rows = reinterpret_cast<uint16_t*>(init_lds + a.Cs);
  const uint64_t st0 = segment_state0(a.seed, b, g, s);
  // the draws do not depend on the shuffle state: j_r = r + (x_r mod (n_s - r))
  for (int r = threadIdx.x; r < cs_eff; r += kInitThreads)
    draw[r] = (uint32_t)r + (uint32_t)(splitmix64_nth(st0, (uint64_t)r) % (uint64_t)(n_s - r));
  for (int i = threadIdx.x; i < n_s; i += kInitThreads) rows[i] = (uint16_t)i;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int r = 0; r < cs_eff; ++r) {
      const int j = (int)draw[r];
      const uint16_t t = rows[r];
      rows[r] = rows[j];
      rows[j] = t;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const T* K = static_cast<const T*>(a.k) + ((size_t)bg * a.N + a.lo + (size_t)s * a.L) * kD;
  T* mh = static_cast<T*>(a.mhat) + ((size_t)bg * a.C + (size_t)s * a.Cs) * kD;
  for (int j = w; j < a.Cs; j += kInitThreads / 64) {
    if (j < cs_eff) {
      const T* row = K + (size_t)rows[j] * kD;
      store_unit_direction<T>((double)St<T>::f(row[2 * lane]), (double)St<T>::f(row[2 * lane + 1]),
                              mh + (size_t)j * kD, buf[w], false);
    } else {
      mh[(size_t)j * kD + 2 * lane] = St<T>::from_f64(0.0);
      mh[(size_t)j * kD + 2 * lane + 1] = St<T>::from_f64(0.0);
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

// a.lo * b.lo + a.hi * b.hi + c for packed bfloat16 pairs: both products are exact in fp32, the
// sums round as fp32 additions.  Emitted directly: the compiler's builtin for this instruction
// picks the wrong 32-bit pieces of a 128-bit register here.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
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
template <typename T, bool kResident>
__global__ __launch_bounds__(assign_threads<T>()) void k_assign(BuildArgs a, int it) {
  extern __shared__ __attribute__((aligned(16))) unsigned char clds[];
  constexpr int CH = AssignCfg<T>::kChunk, STR = AssignCfg<T>::kStride;
  constexpr int NT = assign_threads<T>();          // 64 keys per wave and pass
  const int s = a.seg0 + blockIdx.y, bg = blockIdx.z;
  const int n_s = seg_len_of(a, s);
  const int cs_eff = min(a.Cs, n_s);
  if (blockIdx.x * NT >= n_s) return;
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
  // key (lane & 15) of tile kt; lane group lg holds dims 32 lg .. 32 lg + 31
  constexpr int KE = sizeof(T) == 2 ? 4 : 32;      // bf16: 4 x 8 elements; fp32: 32 elements
  typedef typename std::conditional<sizeof(T) == 2, bf16x8_t, float>::type KElem;
  KElem kb[4][KE];
  // keys past the segment read its last key (in bounds) and are never written back
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int i = min(key0 + w * 64 + kt * 16 + lr, n_s - 1);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < 4; ++st) kb[kt][st] = *reinterpret_cast<const bf16x8_t*>(K + (size_t)i * kD + 32 * lg + 8 * st);
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
        const unsigned char* rp = clds + (ct * 16 + lr) * STR + 64 * lg;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8_t ca = *reinterpret_cast<const bf16x8_t*>(rp + 16 * st);
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
        const u32x4_t cv = *reinterpret_cast<const u32x4_t*>(clds + c * STR + 64 * lg + 16 * st);
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
        const u32x4_t cv = *reinterpret_cast<const u32x4_t*>(mh + (size_t)c * kD + 32 * lg + 8 * st);
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
        const unsigned char* rp = clds + min(4 * grp + r, cs_eff - 1) * STR + 64 * lg;
        f32x4_t dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st)
          dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(rp + 16 * st), kb[kt][st], dd, 0, 0, 0);
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
    if (lane == 0) base = atomicAdd(&a.flag_cnt[it], (uint32_t)__popcll(m));
    base = __builtin_amdgcn_readlane(base, 0);
    if (flagged[kt]) {
      const uint32_t pos = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
      const int i = key0 + w * 64 + kt * 16 + lr;
      a.flag_list[pos] = (int32_t)((size_t)bg * a.Nc + (size_t)s * a.L + i);
    }
  }
  }  // passes
}

// ============================================================================ k_rescore
template <typename T>
__global__ __launch_bounds__(256) void k_rescore(BuildArgs a, int it) {
#pragma clang fp contract(off)
  __shared__ double kx[4][kD];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t n = a.flag_cnt[it];
  for (uint32_t e = blockIdx.x * 4 + w; e < n; e += gridDim.x * 4) {
    const int packed = a.flag_list[e];
    const int bg = packed / a.Nc, ci = packed - bg * a.Nc;
    const int s = ci / a.L;
    const int cs_eff = min(a.Cs, seg_len_of(a, s));
    const T* krow = static_cast<const T*>(a.k) + ((size_t)bg * a.N + a.lo + ci) * kD;
    kx[w][2 * lane] = (double)St<T>::f(krow[2 * lane]);
    kx[w][2 * lane + 1] = (double)St<T>::f(krow[2 * lane + 1]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const T* mh = static_cast<const T*>(a.mhat) + ((size_t)bg * a.C + (size_t)s * a.Cs) * kD;
    double best = -INFINITY;
    int bj = 0x7fffffff;
    for (int j = lane; j < cs_eff; j += 64) {
      const T* crow = mh + (size_t)j * kD;
      double acc = 0.0;
      for (int d0 = 0; d0 < kD; d0 += 8) {
        float cv[8];
        St<T>::load8(crow + d0, cv);
        for (int e2 = 0; e2 < 8; ++e2) {
          const double p = kx[w][d0 + e2] * (double)cv[e2];
          acc = acc + p;
        }
      }
      if (acc > best || bj == 0x7fffffff) { best = acc; bj = j; }
    }
    // wave argmax, ties to the lower id
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
      const double ob = __shfl_xor(best, m);
      const int oj = __shfl_xor(bj, m);
      if (ob > best || (ob == best && oj < bj)) { best = ob; bj = oj; }
    }
    if (lane == 0) a.assign[(size_t)bg * a.Nc + ci] = bj;
    __builtin_amdgcn_wave_barrier();
  }
}

// ============================================================================ k_csr
constexpr int kCsrThreads = 1024;

__global__ __launch_bounds__(kCsrThreads) void k_csr(BuildArgs a) {
  extern __shared__ uint32_t csr_lds[];   // cnt[Cs], loc[Cs], run[Cs], tbl[16][Cs] (u8)
  __shared__ int iscr[32];
  const int s = a.seg0 + blockIdx.x, bg = blockIdx.y;
  const int n_s = seg_len_of(a, s);
  const int Cs = a.Cs;
  uint32_t* cnt = csr_lds;
  uint32_t* loc = csr_lds + Cs;
  uint32_t* run = csr_lds + 2 * Cs;
  uint8_t* tbl = reinterpret_cast<uint8_t*>(csr_lds + 3 * Cs);
  const int32_t* asg = a.assign + (size_t)bg * a.Nc + (size_t)s * a.L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int j = tid; j < Cs; j += kCsrThreads) { cnt[j] = 0u; run[j] = 0u; }
  __syncthreads();
  for (int i = tid; i < n_s; i += kCsrThreads) atomicAdd(&cnt[asg[i]], 1u);
  __syncthreads();
  // exclusive scan of the counts (each thread owns a contiguous run of ids)
  const int per = (Cs + kCsrThreads - 1) / kCsrThreads;
  const int j0 = min(Cs, tid * per), j1 = min(Cs, j0 + per);
  int my = 0;
  for (int j = j0; j < j1; ++j) my += (int)cnt[j];
  int tot;
  int ex = block_exclusive_scan<kCsrThreads>(my, iscr, &tot);
  for (int j = j0; j < j1; ++j) { loc[j] = (uint32_t)ex; ex += (int)cnt[j]; }
  __syncthreads();
  const int cbase = s * Cs;
  for (int j = tid; j < Cs; j += kCsrThreads) {
    a.sizes[(size_t)bg * a.C + cbase + j] = (int32_t)cnt[j];
    a.offsets[(size_t)bg * (a.C + 1) + cbase + j] = s * a.L + (int32_t)loc[j];
  }
  // stable scatter: rounds of 1024 tokens in order; within a wave, lanes with equal ids are
  // ranked by lane; across waves of a round by the per-wave count table; across rounds by run[].
  int32_t* perm = a.perm + (size_t)bg * a.Nc + (size_t)s * a.L;
  const int pos0 = a.lo + s * a.L;
  for (int r0 = 0; r0 < n_s; r0 += kCsrThreads) {
    for (int x = tid; x < 16 * Cs / 4; x += kCsrThreads) reinterpret_cast<uint32_t*>(tbl)[x] = 0u;
    __syncthreads();
    const int i = r0 + tid;
    const bool valid = i < n_s;
    const int key = valid ? asg[i] : -1;
    uint64_t mine = 0;
    for (int j = 0; j < 64; ++j) {
      const int sk = __builtin_amdgcn_readlane(key, j);
      const uint64_t m = __ballot(key == sk);
      if (key == sk) mine = m;
    }
    const int rank = __popcll(mine & ((1ull << lane) - 1ull));
    if (valid && rank == 0) tbl[w * Cs + key] = (uint8_t)__popcll(mine);
    __syncthreads();
    if (valid) {
      int p = (int)loc[key] + (int)run[key] + rank;
      for (int ww = 0; ww < w; ++ww) p += tbl[ww * Cs + key];
      perm[p] = pos0 + i;
    }
    __syncthreads();
    for (int j = tid; j < Cs; j += kCsrThreads) {
      uint32_t add = 0;
      for (int ww = 0; ww < 16; ++ww) add += tbl[ww * Cs + j];
      run[j] += add;
    }
    __syncthreads();
  }
}

// ============================================================================ k_update / k_final
// One wave per cluster; lane owns dims 2*lane, 2*lane+1.  Members are summed in fp64 in
// ascending position (the CSR order), 16 rows fetched ahead of the sums.
template <typename T, bool kFinal>
__global__ __launch_bounds__(512) void k_sums(BuildArgs a) {
  __shared__ double buf[8][kD];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int s = a.seg0 + blockIdx.y, bg = blockIdx.z;
  const int j = blockIdx.x * 8 + w;
  if (j >= a.Cs) return;
  const int n_s = seg_len_of(a, s);
  const int cs_eff = min(a.Cs, n_s);
  const int c = s * a.Cs + j;
  const size_t cidx = (size_t)bg * a.C + c;
  T* dst = static_cast<T*>(kFinal ? a.mu : a.mhat) + cidx * kD;
  if (j >= cs_eff) {
    if (kFinal) {
      T* sv = static_cast<T*>(a.sv) + cidx * kD;
      dst[2 * lane] = St<T>::from_f64(0.0); dst[2 * lane + 1] = St<T>::from_f64(0.0);
      sv[2 * lane] = St<T>::from_f64(0.0); sv[2 * lane + 1] = St<T>::from_f64(0.0);
    }
    return;
  }
  const int n = a.sizes[cidx];
  const int start = a.offsets[(size_t)bg * (a.C + 1) + c];
  const int32_t* perm = a.perm + (size_t)bg * a.Nc;
  const T* K = static_cast<const T*>(a.k) + (size_t)bg * a.N * kD;
  const T* V = static_cast<const T*>(a.v) + (size_t)bg * a.N * kD;
  T* kp = static_cast<T*>(a.kp) + (size_t)bg * a.Nc * kD;
  T* vp = static_cast<T*>(a.vp) + (size_t)bg * a.Nc * kD;
  double k0 = 0.0, k1 = 0.0, v0 = 0.0, v1 = 0.0;
  for (int m0 = 0; m0 < n; m0 += 16) {
    const int cnt = min(16, n - m0);
    int p = 0;
    if (lane < cnt) p = perm[start + m0 + lane];
    T kx[16][2], vx[16][2];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int pos = __shfl(p, u);
      if (u < cnt) {
        kx[u][0] = K[(size_t)pos * kD + 2 * lane];
        kx[u][1] = K[(size_t)pos * kD + 2 * lane + 1];
        if (kFinal) {
          vx[u][0] = V[(size_t)pos * kD + 2 * lane];
          vx[u][1] = V[(size_t)pos * kD + 2 * lane + 1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u < cnt) {
#pragma clang fp contract(off)
        k0 = k0 + (double)St<T>::f(kx[u][0]);
        k1 = k1 + (double)St<T>::f(kx[u][1]);
        if (kFinal) {
          v0 = v0 + (double)St<T>::f(vx[u][0]);
          v1 = v1 + (double)St<T>::f(vx[u][1]);
          const size_t r = (size_t)(start + m0 + u) * kD;
          kp[r + 2 * lane] = kx[u][0]; kp[r + 2 * lane + 1] = kx[u][1];
          vp[r + 2 * lane] = vx[u][0]; vp[r + 2 * lane + 1] = vx[u][1];
        }
      }
    }
  }
  if (kFinal) {
    T* sv = static_cast<T*>(a.sv) + cidx * kD;
    if (n > 0) {
      const double dn = (double)n;
      dst[2 * lane] = St<T>::from_f64(k0 / dn);
      dst[2 * lane + 1] = St<T>::from_f64(k1 / dn);
      sv[2 * lane] = St<T>::from_f64(v0);
      sv[2 * lane + 1] = St<T>::from_f64(v1);
    } else {
      dst[2 * lane] = St<T>::from_f64(0.0); dst[2 * lane + 1] = St<T>::from_f64(0.0);
      sv[2 * lane] = St<T>::from_f64(0.0); sv[2 * lane + 1] = St<T>::from_f64(0.0);
    }
  } else if (n > 0) {
    store_unit_direction<T>(k0, k1, dst, buf[w], true);
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
    const size_t lds = (size_t)a.Cs * 4 + (((size_t)a.L * 2 + 3) & ~size_t(3));
    prof_begin(WI_STAGE_INIT, st);
    hipLaunchKernelGGL(k_init<T>, dim3(nseg_b, BG), dim3(kInitThreads), lds, st, a);
    prof_end(WI_STAGE_INIT, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t alds = (size_t)AssignCfg<T>::kChunk * AssignCfg<T>::kStride;
  const size_t clds = (size_t)a.Cs * 12 + (size_t)16 * a.Cs;
  // assignment blocks per segment: about one block per CU in all (each stages the segment's
  // centroids once and loops over 64-key-per-wave passes), at least one pass each
  const unsigned assign_px = (unsigned)std::max<int64_t>(1, std::min<int64_t>(
      ceil_div(a.L, assign_threads<T>()), ceil_div(kAssignBlocksTarget, (int64_t)nseg_b * BG)));
  for (int it = 0; it < a.iters; ++it) {
    prof_begin(WI_STAGE_ASSIGN, st);
    if (a.Cs <= AssignCfg<T>::kChunk)
      hipLaunchKernelGGL((k_assign<T, true>), dim3(assign_px, nseg_b, BG), dim3(assign_threads<T>()),
                         alds, st, a, it);
    else
      hipLaunchKernelGGL((k_assign<T, false>), dim3(assign_px, nseg_b, BG), dim3(assign_threads<T>()),
                         alds, st, a, it);
    prof_end(WI_STAGE_ASSIGN, st);
    prof_begin(WI_STAGE_RESCORE, st);
    hipLaunchKernelGGL(k_rescore<T>, dim3(1024), dim3(256), 0, st, a, it);
    prof_end(WI_STAGE_RESCORE, st);
    prof_begin(WI_STAGE_CSR, st);
    hipLaunchKernelGGL(k_csr, dim3(nseg_b, BG), dim3(kCsrThreads), clds, st, a);
    prof_end(WI_STAGE_CSR, st);
    if (it + 1 < a.iters) {
      prof_begin(WI_STAGE_UPDATE, st);
      hipLaunchKernelGGL((k_sums<T, false>), dim3((unsigned)ceil_div(a.Cs, 8), nseg_b, BG), dim3(512), 0, st, a);
      prof_end(WI_STAGE_UPDATE, st);
    } else {
      prof_begin(WI_STAGE_FINAL, st);
      hipLaunchKernelGGL((k_sums<T, true>), dim3((unsigned)ceil_div(a.Cs, 8), nseg_b, BG), dim3(512), 0, st, a);
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
