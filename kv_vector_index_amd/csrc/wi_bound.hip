// Per-cluster data of the estimation error bound: the radius of every cluster around its stored
// mean key, the largest value norm of its members, and the largest value norm of the context.
//
// The pages promise a controlled error for the estimation zone (RetroInfer technical summary,
// section 2.A item 3; Arabic summary, section 2.a, accuracy-bound estimation) without a formula.
// The bound used here brackets each member's softmax weight exp(s <q, k_i>) within
// exp(+-s |q| r_c) of the centroid's weight exp(s <q, mu_c>), r_c = max |k_i - mu_c|; the decode
// kernels turn r_c, the value norms and the stored sums' rounding into a bound on the output.
//
// Definitions, identical in the oracle: |x|^2 is the sum over coordinates in ascending order of
// the fp64 squares (a difference k_ij - mu_cj rounded to fp64 first, each square and each add
// rounded, no fused multiply-add); the cluster's figure is the maximum over its members, and the
// stored value is the smallest fp32 f >= 0 with f * f >= that maximum (its square root rounded up;
// f * f is exact in fp64, so the test is exact).  Taking the maximum of the rounded-up roots is the
// same, so every row folds its own figure in with an atomic maximum on the fp32 bit pattern
// (non-negative floats order like their bits), and the result does not depend on the order.
#include "wi_device.h"
#include "wi_internal.h"

namespace wi {

constexpr int kBoundThreads = 256;

// sum over j ascending of x_j^2, x_j = a_j - b_j (b null: x = a), in fp64 without contraction
template <typename T>
__device__ __forceinline__ double row_sq_norm(const T* __restrict__ a, const T* __restrict__ b) {
#pragma clang fp contract(off)
  double acc = 0.0;
  for (int j0 = 0; j0 < kD; j0 += 8) {
    float x[8], y[8];
    St<T>::load8(a + j0, x);
    if (b) St<T>::load8(b + j0, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double t = b ? (double)x[e] - (double)y[e] : (double)x[e];
      const double sq = t * t;
      acc = acc + sq;
    }
  }
  return acc;
}

// smallest fp32 f >= 0 with (double)f * f >= d2 (d2 >= 0)
__device__ __forceinline__ float sqrt_up_f32(double d2) {
  float f = (float)sqrt(d2);
  if ((double)f * (double)f < d2) {
    f = nextafterf(f, INFINITY);
  } else {
    while (f > 0.f) {
      const float p = nextafterf(f, 0.f);
      if ((double)p * (double)p < d2) break;
      f = p;
    }
  }
  return f;
}

__global__ __launch_bounds__(kBoundThreads) void k_bound_zero(float* radius, float* vnorm, float* vmax,
                                                              int64_t n_clusters, int64_t n_groups) {
  const int64_t i = (int64_t)blockIdx.x * kBoundThreads + threadIdx.x;
  if (i < n_clusters) { radius[i] = 0.f; vnorm[i] = 0.f; }
  if (i < n_groups) vmax[i] = 0.f;
}

// thread -> one row of (b, g) = blockIdx.y: clustered rows [0, Nc) then steady rows [Nc, Nc + NS)
template <typename T>
__global__ __launch_bounds__(kBoundThreads) void k_bound_data(const T* __restrict__ mu, const int32_t* __restrict__ offsets,
                                                              const T* __restrict__ k_perm, const T* __restrict__ v_perm,
                                                              const T* __restrict__ v_steady, int C, int Nc, int NS,
                                                              float* radius, float* vnorm, float* vmax) {
  const int bg = blockIdx.y;
  const int r = blockIdx.x * kBoundThreads + threadIdx.x;
  if (r >= Nc + NS) return;
  unsigned* vmax_bits = reinterpret_cast<unsigned*>(vmax) + bg;
  if (r >= Nc) {
    const T* v = v_steady + ((size_t)bg * NS + (r - Nc)) * kD;
    atomicMax(vmax_bits, __float_as_uint(sqrt_up_f32(row_sq_norm<T>(v, nullptr))));
    return;
  }
  // the cluster owning row r: the last c with offsets[c] <= r (a non-empty one)
  const int32_t* off = offsets + (size_t)bg * (C + 1);
  int lo = 0, hi = C;                           // off[lo] <= r < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid;
  }
  const size_t row = (size_t)bg * Nc + r;
  const float rk = sqrt_up_f32(row_sq_norm<T>(k_perm + row * kD, mu + ((size_t)bg * C + lo) * kD));
  const float rv = sqrt_up_f32(row_sq_norm<T>(v_perm + row * kD, nullptr));
  atomicMax(reinterpret_cast<unsigned*>(radius) + (size_t)bg * C + lo, __float_as_uint(rk));
  atomicMax(reinterpret_cast<unsigned*>(vnorm) + (size_t)bg * C + lo, __float_as_uint(rv));
  atomicMax(vmax_bits, __float_as_uint(rv));
}

hipError_t launch_bound_data(const wi_decode_params& p, const wi_index_view& idx, float* radius, float* vnorm,
                             float* vmax, hipStream_t s) {
  const int BG = p.B * p.Hkv;
  const int64_t nc = (int64_t)BG * p.C;
  const int64_t nz = std::max<int64_t>(nc, BG);
  hipLaunchKernelGGL(k_bound_zero, dim3((unsigned)ceil_div(nz, kBoundThreads)), dim3(kBoundThreads), 0, s,
                     radius, vnorm, vmax, nc, (int64_t)BG);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.Nc + p.n_steady;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(rows, kBoundThreads), BG);
  if (p.dtype == WI_BF16)
    hipLaunchKernelGGL(k_bound_data<uint16_t>, grid, dim3(kBoundThreads), 0, s,
                       static_cast<const uint16_t*>(idx.centroids), idx.offsets,
                       static_cast<const uint16_t*>(idx.k_perm), static_cast<const uint16_t*>(idx.v_perm),
                       static_cast<const uint16_t*>(idx.v_steady), p.C, p.Nc, p.n_steady, radius, vnorm, vmax);
  else
    hipLaunchKernelGGL(k_bound_data<float>, grid, dim3(kBoundThreads), 0, s,
                       static_cast<const float*>(idx.centroids), idx.offsets,
                       static_cast<const float*>(idx.k_perm), static_cast<const float*>(idx.v_perm),
                       static_cast<const float*>(idx.v_steady), p.C, p.Nc, p.n_steady, radius, vnorm, vmax);
  return hipGetLastError();
}

}  // namespace wi
