// Device-side helpers shared by the wave-index kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wi {

constexpr int kD = 128;     // head dimension the kernels are written for
constexpr int kWave = 64;   // CDNA wavefront width

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ element conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Storage traits: float (fp32) or uint16_t (bf16 bits).
template <typename T> struct St;
template <> struct St<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float f(float x) { return x; }
  // fp64 -> fp32 by round-to-nearest-even
  __device__ __forceinline__ static float from_f64(double x) { return (float)x; }
  // 8 consecutive elements starting at p (32-byte aligned)
  __device__ __forceinline__ static void load8(const float* p, float (&o)[8]) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p + 4);
    o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y);
    o[2] = __uint_as_float(a.z); o[3] = __uint_as_float(a.w);
    o[4] = __uint_as_float(b.x); o[5] = __uint_as_float(b.y);
    o[6] = __uint_as_float(b.z); o[7] = __uint_as_float(b.w);
  }
};
template <> struct St<uint16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float f(uint16_t x) { return bf16_bits_to_f32(x); }
  // fp64 -> fp32 (RNE) -> bf16 (RNE): two rounding steps
  __device__ __forceinline__ static uint16_t from_f64(double x) { return f32_to_bf16_bits((float)x); }
  __device__ __forceinline__ static void load8(const uint16_t* p, float (&o)[8]) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
    o[0] = __uint_as_float(a.x << 16); o[1] = __uint_as_float(a.x & 0xffff0000u);
    o[2] = __uint_as_float(a.y << 16); o[3] = __uint_as_float(a.y & 0xffff0000u);
    o[4] = __uint_as_float(a.z << 16); o[5] = __uint_as_float(a.z & 0xffff0000u);
    o[6] = __uint_as_float(a.w << 16); o[7] = __uint_as_float(a.w & 0xffff0000u);
  }
};

// fp32 -> uint32 whose unsigned order is the float order (-NaN < -Inf < ... < +Inf < +NaN).
// a.lo * b.lo + a.hi * b.hi + c for packed bfloat16 pairs: both products are exact in fp32, the
// sums round as fp32 additions.  Emitted directly: the compiler's builtin for this instruction
// picks the wrong 32-bit pieces of a 128-bit register.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ uint64_t f64_order_key(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Orders this wave's LDS writes before its later LDS reads (and the reverse) without a block
// barrier: the lanes of one wave hand values to each other through LDS.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A zero the compiler cannot see through.  Indexing an LDS array of loop-invariant values with it
// inside a loop keeps the compiler from hoisting all of those values into registers ahead of the
// loop (they would not fit and would be spilled to scratch memory).
__device__ __forceinline__ int opaque_zero() {
  int z = 0;
  asm volatile("" : "+v"(z));
  return z;
}

// ------------------------------------------------------------------ wave / block reductions
// Lane exchanges inside a DPP row of 16 lanes (VALU operand modifiers, no LDS traffic):
// quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140, row_shr:n = 0x110 + n (lanes shifted in from outside the row read 0).
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, true); }
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) { return __int_as_float(dpp_i<kCtrl>(__float_as_int(v))); }
__device__ __forceinline__ float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

// All-lane reductions: a butterfly inside each row, then the four row results combined in a
// fixed order ((row 0, row 1), (row 2, row 3)).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ int wave_isum(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x141>(v);
  v += dpp_i<0x140>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  int x = (int)v;
  x = (int)max((uint32_t)x, (uint32_t)dpp_i<0xB1>(x));
  x = (int)max((uint32_t)x, (uint32_t)dpp_i<0x4E>(x));
  x = (int)max((uint32_t)x, (uint32_t)dpp_i<0x141>(x));
  x = (int)max((uint32_t)x, (uint32_t)dpp_i<0x140>(x));
  return max(max((uint32_t)__builtin_amdgcn_readlane(x, 0), (uint32_t)__builtin_amdgcn_readlane(x, 16)),
             max((uint32_t)__builtin_amdgcn_readlane(x, 32), (uint32_t)__builtin_amdgcn_readlane(x, 48)));
}

// Inclusive prefix sum within a wave: Hillis-Steele inside each row (shifts 1, 2, 4, 8), then
// the totals of the lower rows added.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp_i<0x111>(v);
  v += dpp_i<0x112>(v);
  v += dpp_i<0x114>(v);
  v += dpp_i<0x118>(v);
  const int s1 = __builtin_amdgcn_readlane(v, 15);
  const int s2 = __builtin_amdgcn_readlane(v, 31);
  const int s3 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? s1 : 0) + (row >= 2 ? s2 : 0) + (row >= 3 ? s3 : 0);
}

// The same for floats (the additions of a scan: any order is fine where this is used).
__device__ __forceinline__ float wave_inclusive_scan_f(float v) {
  v += dpp_f<0x111>(v);
  v += dpp_f<0x112>(v);
  v += dpp_f<0x114>(v);
  v += dpp_f<0x118>(v);
  const float s1 = readlane_f(v, 15);
  const float s2 = readlane_f(v, 31);
  const float s3 = readlane_f(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? s1 : 0.f) + (row >= 2 ? s2 : 0.f) + (row >= 3 ? s3 : 0.f);
}

// Block-wide scans and reductions over NT threads (a multiple of 64, <= 1024; NT is the launch
// block size, a compile-time constant so that no work-group size is read at run time).  `scratch`
// holds >= NT / 64 entries of LDS; every thread reads all per-wave partials itself.

// Exclusive prefix sum: returns this thread's exclusive prefix; *total receives the block sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  constexpr int nw = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < nw; ++i) {
    const int t = scratch[i];
    before += i < w ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return before + inc - v;
}

template <int NT>
__device__ __forceinline__ float block_exclusive_scan_f(float v, float* scratch, float* total) {
  constexpr int nw = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float inc = wave_inclusive_scan_f(v);
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  float before = 0.f, tot = 0.f;
#pragma unroll
  for (int i = 0; i < nw; ++i) {
    const float t = scratch[i];
    before += i < w ? t : 0.f;
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return before + (inc - v);
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* scratch) {
  constexpr int nw = NT / 64;
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < nw; ++i) r = fmaxf(r, scratch[i]);
  __syncthreads();
  return r;
}
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* scratch) {
  constexpr int nw = NT / 64;
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < nw; ++i) r += scratch[i];
  __syncthreads();
  return r;
}
template <int NT>
__device__ __forceinline__ int block_isum(int v, int* scratch) {
  constexpr int nw = NT / 64;
  v = wave_isum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < nw; ++i) r += scratch[i];
  __syncthreads();
  return r;
}

}  // namespace wi
