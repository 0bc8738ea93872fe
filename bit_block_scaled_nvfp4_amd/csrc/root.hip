// root.hip -- the pieces of the Newton-Schulz orthogonalization run in NVFP4
// ("Full-Stack FP4 ...", section 2.3, Q-Root) that are not a quantize or a
// GEMM: the exact order statistic of |x| used as the outlier clip (a radix
// select over the FP32 bit patterns of |x|, three digit passes), and the
// Frobenius normalization of the input.
//
// Radix select.  For x >= 0 the IEEE bit patterns order like the values
// (NaN patterns above +inf), so the k-th smallest |x| is found digit by
// digit on u = bits(x) & 0x7FFFFFFF: bits 30..19 (12), 18..8 (11), 7..0 (8).
// Pass p histograms digit p of the elements whose higher digits equal the
// prefix found so far (LDS bins per workgroup, one global atomic add per
// nonzero bin), then one workgroup scans the histogram, narrows the prefix
// and the rank left inside it, and clears the histogram for the next pass or
// call.  Counts are exact integers, so the result does not depend on the
// order of the atomics.  The first digit is the widest: every element
// counts in that pass, and real data crowd into a few exponents, whose bins
// the LDS atomics then serialize on.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"

namespace nvfp4 {
namespace {

constexpr int kSelThreads = 256;
constexpr int kBins = 4096;  // the widest digit's bins (the histogram's size)

// Digit widths and positions: pass 0 bits 30..19, pass 1 bits 18..8, pass 2
// bits 7..0.
constexpr int kDigitBits[3] = {12, 11, 8};
constexpr int kDigitShift[3] = {19, 8, 0};

__device__ __forceinline__ uint32_t abs_u(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

template <int kPass>
__device__ __forceinline__ uint32_t digit(uint32_t u) {
  return (u >> kDigitShift[kPass]) & ((1u << kDigitBits[kPass]) - 1u);
}

// The higher digits of u, compared with the prefix of pass kPass.
template <int kPass>
__device__ __forceinline__ bool in_prefix(uint32_t u, uint32_t prefix) {
  if constexpr (kPass == 0) return true;
  else return (u >> kDigitShift[kPass - 1]) == prefix;
}

struct SelArgs {
  const float *x;
  int64_t rows, cols, ld;   // [rows][cols], row stride ld; cols % 4 == 0, ld % 4 == 0
  SelectState *state;
  uint32_t *hist;           // kBins counters, zero on entry
};

template <int kPass>
__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(SelArgs a) {
  constexpr int kN = 1 << kDigitBits[kPass];
  __shared__ uint32_t bins[kN];
  for (int i = threadIdx.x; i < kN; i += kSelThreads) bins[i] = 0u;
  __syncthreads();
  const uint32_t prefix = kPass == 0 ? 0u : a.state->prefix;
  const uint64_t vpr = (uint64_t)(a.cols / 4);  // float4 per row
  const uint64_t nvec = (uint64_t)a.rows * vpr;
  for (uint64_t v = (uint64_t)blockIdx.x * kSelThreads + threadIdx.x; v < nvec;
       v += (uint64_t)gridDim.x * kSelThreads) {
    const uint64_t r = v / vpr, c4 = v - r * vpr;
    const float4 q = *reinterpret_cast<const float4 *>(a.x + r * a.ld + 4 * c4);
    const uint32_t u[4] = {abs_u(q.x), abs_u(q.y), abs_u(q.z), abs_u(q.w)};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (in_prefix<kPass>(u[i], prefix)) atomicAdd(&bins[digit<kPass>(u[i])], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kN; i += kSelThreads)
    if (bins[i]) atomicAdd(&a.hist[i], bins[i]);
}

// One workgroup: find the bin holding rank `rank` (0-based, ascending) among
// this pass's elements, narrow the prefix, and clear the histogram.  On the
// last pass the prefix is the whole pattern: store the value.
template <int kPass>
__global__ __launch_bounds__(kSelThreads) void select_scan_kernel(SelectState *st, uint32_t *hist, uint64_t rank0) {
  constexpr int kPer = (1 << kDigitBits[kPass]) / kSelThreads;  // bins per thread
  __shared__ uint64_t part[kSelThreads];
  const uint64_t rank = kPass == 0 ? rank0 : st->rank;
  uint32_t c[kPer];
  uint64_t sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    c[i] = hist[threadIdx.x * kPer + i];
    sum += c[i];
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  // Inclusive scan over the 256 partial sums (Hillis-Steele in LDS).
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const uint64_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0ull;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  const uint64_t before = threadIdx.x ? part[threadIdx.x - 1] : 0ull;
  if (rank >= before && rank < part[threadIdx.x]) {
    // This thread's bins hold the rank: the first bin whose running count
    // passes it.
    uint64_t below = before;
    int b = -1;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (b < 0 && rank < below + c[i]) b = i;
      if (b < 0) below += c[i];
    }
    const uint32_t d = (uint32_t)(threadIdx.x * kPer + b);
    const uint32_t prefix = kPass == 0 ? d : ((st->prefix << kDigitBits[kPass]) | d);
    st->prefix = prefix;
    st->rank = rank - below;
    if (kPass == 2) st->value = __uint_as_float(prefix);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) hist[threadIdx.x * kPer + i] = 0u;
}

// Frobenius normalization: per-workgroup FP64 sums of squares, one
// workgroup adds the partials in index order and stores 1 / (||g|| + eps)
// rounded to FP32, then every element is scaled by it.
constexpr int kNormGroups = 1024;

struct NormArgs {
  const void *g;
  bool bf16;
  int64_t rows, cols, ld;  // cols % 4 == 0, ld % 4 == 0
  double *partial;         // kNormGroups
  float *inv;              // 1 / (||g||_F + eps)
  float *x;                // [rows][cols] FP32, row stride xld
  int64_t xld;
};

__device__ __forceinline__ float4 load4(const NormArgs &a, uint64_t r, uint64_t c4) {
  if (a.bf16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.g) + r * a.ld + 4 * c4);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xFFFF0000u));
  }
  return *reinterpret_cast<const float4 *>(static_cast<const float *>(a.g) + r * a.ld + 4 * c4);
}

__global__ __launch_bounds__(kSelThreads) void norm_partial_kernel(NormArgs a) {
  __shared__ double red[kSelThreads];
  const uint64_t vpr = (uint64_t)(a.cols / 4);
  const uint64_t nvec = (uint64_t)a.rows * vpr;
  double s = 0.0;
  for (uint64_t v = (uint64_t)blockIdx.x * kSelThreads + threadIdx.x; v < nvec;
       v += (uint64_t)gridDim.x * kSelThreads) {
    const uint64_t r = v / vpr, c4 = v - r * vpr;
    const float4 q = load4(a, r, c4);
    s += (double)q.x * q.x + (double)q.y * q.y + (double)q.z * q.z + (double)q.w * q.w;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = kSelThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kSelThreads) void norm_finish_kernel(NormArgs a, int ngroups) {
  __shared__ double red[kSelThreads];
  double s = 0.0;
  for (int i = threadIdx.x; i < ngroups; i += kSelThreads) s += a.partial[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = kSelThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *a.inv = (float)(1.0 / (sqrt(red[0]) + 1e-7));
}

__global__ __launch_bounds__(kSelThreads) void norm_scale_kernel(NormArgs a) {
  const float inv = *a.inv;
  const uint64_t vpr = (uint64_t)(a.cols / 4);
  const uint64_t nvec = (uint64_t)a.rows * vpr;
  for (uint64_t v = (uint64_t)blockIdx.x * kSelThreads + threadIdx.x; v < nvec;
       v += (uint64_t)gridDim.x * kSelThreads) {
    const uint64_t r = v / vpr, c4 = v - r * vpr;
    const float4 q = load4(a, r, c4);
    *reinterpret_cast<float4 *>(a.x + r * a.xld + 4 * c4) = make_float4(q.x * inv, q.y * inv, q.z * inv, q.w * inv);
  }
}

int stride_grid(uint64_t nvec, uint64_t cap) {
  const uint64_t g = (nvec + kSelThreads - 1) / kSelThreads;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

nvfp4_status launch_abs_select(const float *x, int64_t rows, int64_t cols, int64_t ld, uint64_t rank,
                               SelectState *state, uint32_t *hist, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return NVFP4_EINVAL;
  SelArgs a{x, rows, cols, ld, state, hist};
  const int g = stride_grid((uint64_t)rows * (uint64_t)(cols / 4), 2048);
  hipLaunchKernelGGL(select_hist_kernel<0>, dim3(g), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_scan_kernel<0>, dim3(1), dim3(kSelThreads), 0, s, state, hist, rank);
  hipLaunchKernelGGL(select_hist_kernel<1>, dim3(g), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_scan_kernel<1>, dim3(1), dim3(kSelThreads), 0, s, state, hist, rank);
  hipLaunchKernelGGL(select_hist_kernel<2>, dim3(g), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_scan_kernel<2>, dim3(1), dim3(kSelThreads), 0, s, state, hist, rank);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status launch_frobenius_normalize(const void *g, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                                        double *partial, float *inv, float *x, int64_t xld, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return NVFP4_EINVAL;
  NormArgs a{g, bf16, rows, cols, ld, partial, inv, x, xld};
  const uint64_t nvec = (uint64_t)rows * (uint64_t)(cols / 4);
  hipLaunchKernelGGL(norm_partial_kernel, dim3(kNormGroups), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(norm_finish_kernel, dim3(1), dim3(kSelThreads), 0, s, a, kNormGroups);
  hipLaunchKernelGGL(norm_scale_kernel, dim3(stride_grid(nvec, 8192)), dim3(kSelThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace nvfp4
