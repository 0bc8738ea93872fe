// root.hip -- the pieces of the Newton-Schulz orthogonalization run in NVFP4
// ("Full-Stack FP4 ...", section 2.3, Q-Root) that are not a quantize or a
// GEMM: the exact order statistic of |x| used as the outlier clip (a radix
// select over the FP32 bit patterns of |x|, three digit passes), and the
// Frobenius normalization of the input.
//
// Radix select.  For x >= 0 the IEEE bit patterns order like the values
// (NaN patterns above +inf), so the k-th smallest |x| is found digit by
// digit on the keys u = bits(x) & 0x7FFFFFFF, taken relative to a base
// (d = u - base, of which the low W bits vary): digits of up to 12, 12 and 8
// bits from the top of those W bits.  Pass p histograms digit p of the keys
// whose higher digits equal the prefix found so far (LDS bins per workgroup,
// one global atomic add per nonzero bin), then one workgroup scans the
// histogram, narrows the prefix and the rank left inside it, and clears the
// histogram for the next pass or call.  Counts are exact integers, so the
// result does not depend on the order of the atomics.
//
// Sampled bracket.  Before the digit passes, one workgroup sorts 1024 keys
// sampled at evenly spaced positions and takes the keys 24 sample ranks
// either side of the target's sample rank as a bracket [lo, hi]; one pass
// over the tensor counts the keys below lo and copies the keys inside the
// bracket to a compact buffer (about 5% of them), staged per workgroup in
// LDS so that each workgroup reserves its space with one atomic.  If the
// target rank falls inside the bracket, the digit passes run over the
// compact copy for the rank relative to it, with base lo and W the width of
// hi - lo: the first digit then spreads the bracket's keys over up to 4096
// bins, where digits of u itself would crowd them into the few exponents
// they share.  Otherwise (a bracket that missed, or more keys than the
// buffer holds) they run over the tensor with base 0 and W = 31.  Either way
// the result is the exact order statistic; the sample only decides how much
// the digit passes read.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"

namespace nvfp4 {
namespace {

constexpr int kSelThreads = 256;
constexpr int kBins = 4096;  // the widest digit's bins (the histogram's size)

__device__ __forceinline__ uint32_t abs_u(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// Element offset of float4 number v of a tensor with vpr float4 per row and
// row stride ld: 4 v where the rows are contiguous, else through the row
// index (a 64-bit division, which would otherwise cost more than the rest of
// these memory-bound loops).
__device__ __forceinline__ uint64_t vec_off(uint64_t v, uint64_t vpr, int64_t ld) {
  if ((uint64_t)ld == 4 * vpr) return 4 * v;
  const uint64_t r = v / vpr;
  return r * (uint64_t)ld + 4 * (v - r * vpr);
}

struct SelArgs {
  const float *x;
  int64_t rows, cols, ld;   // [rows][cols], row stride ld; cols % 4 == 0, ld % 4 == 0
  SelectState *state;
  uint32_t *hist;           // kBins counters, zero on entry
  uint32_t *compact;        // the bracket's keys
  uint64_t cap;             // capacity of `compact`
};

constexpr int kSampleThreads = 512;
constexpr int kSamples = 1024;   // sorted in LDS by one workgroup
constexpr int kMargin = 24;      // sample ranks either side of the target's (7.5 standard deviations at p99)

// Element (flat index i of [rows][cols]) as its key.
__device__ __forceinline__ uint32_t key_at(const SelArgs &a, uint64_t i) {
  if (a.ld == a.cols) return abs_u(a.x[i]);
  const uint64_t r = i / (uint64_t)a.cols, c = i - r * (uint64_t)a.cols;
  return abs_u(a.x[r * a.ld + c]);
}

__global__ __launch_bounds__(kSampleThreads) void select_sample_kernel(SelArgs a, uint64_t rank) {
  __shared__ uint32_t k[kSamples];
  SelectState *st = a.state;
  const uint64_t n = (uint64_t)a.rows * (uint64_t)a.cols;
  for (int i = threadIdx.x; i < kSamples; i += kSampleThreads) k[i] = key_at(a, (uint64_t)i * n / kSamples);
  __syncthreads();
  // bitonic sort, ascending: at each stage every thread takes whole
  // compare-exchange pairs (i, i + stride)
  for (int size = 2; size <= kSamples; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = threadIdx.x; p < kSamples / 2; p += kSampleThreads) {
        const int i = ((p & ~(stride - 1)) << 1) | (p & (stride - 1)), j = i + stride;  // stride: a power of 2
        const uint32_t x = k[i], y = k[j];
        const bool up = (i & size) == 0;
        if ((x > y) == up) {
          k[i] = y;
          k[j] = x;
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    const int64_t ks = (int64_t)(rank * kSamples / n);
    st->lo = ks - kMargin <= 0 ? 0u : k[ks - kMargin];
    st->hi = ks + kMargin >= kSamples - 1 ? 0xFFFFFFFFu : k[ks + kMargin];
    st->below = 0ull;
    st->count = 0u;
    st->overflow = 0u;
    st->rank0 = rank;
    st->mode = 1u;
  }
}

// One pass over the tensor: keys below the bracket counted, keys inside it
// copied out.  One workgroup per CU (few global atomics on the two shared
// counters, whose same-address updates serialize), four 16-byte loads per
// thread in flight per round.  A workgroup stages its bracket keys in LDS
// (an LDS atomic per key; they are about 5% of the keys) and at the end
// reserves their place in the compact buffer with one global atomic; keys
// beyond the staging space go straight out, one global atomic each.
constexpr int kBracketThreads = 1024;
constexpr int kBracketUnroll = 4;
constexpr int kBracketKeys = 8192;

__global__ __launch_bounds__(kBracketThreads) void select_bracket_kernel(SelArgs a) {
  __shared__ uint32_t lbuf[kBracketKeys];
  __shared__ uint32_t lcount, gbase;
  __shared__ unsigned long long red[kBracketThreads / 64];
  SelectState *st = a.state;
  if (threadIdx.x == 0) lcount = 0u;
  __syncthreads();
  const uint32_t lo = st->lo, hi = st->hi;
  const uint64_t vpr = (uint64_t)(a.cols / 4);
  const uint64_t nvec = (uint64_t)a.rows * vpr;
  const uint64_t stride = (uint64_t)gridDim.x * kBracketThreads;
  uint32_t below = 0;
  for (uint64_t v0 = (uint64_t)blockIdx.x * kBracketThreads + threadIdx.x; v0 < nvec;
       v0 += kBracketUnroll * stride) {
    float4 q[kBracketUnroll];
#pragma unroll
    for (int t = 0; t < kBracketUnroll; ++t) {
      // past the end: a clamped (in-bounds) load, masked below
      const uint64_t v = min(v0 + t * stride, nvec - 1);
      q[t] = *reinterpret_cast<const float4 *>(a.x + vec_off(v, vpr, a.ld));
    }
#pragma unroll
    for (int t = 0; t < kBracketUnroll; ++t) {
      if (v0 + t * stride >= nvec) break;
      const uint32_t u[4] = {abs_u(q[t].x), abs_u(q[t].y), abs_u(q[t].z), abs_u(q[t].w)};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        below += u[i] < lo ? 1u : 0u;
        if (u[i] >= lo && u[i] <= hi) {
          const uint32_t slot = atomicAdd(&lcount, 1u);
          if (slot < kBracketKeys) {
            lbuf[slot] = u[i];
          } else {
            const uint32_t pos = atomicAdd(&st->count, 1u);
            if (pos < a.cap) a.compact[pos] = u[i];
            else st->overflow = 1u;
          }
        }
      }
    }
  }
  // the workgroup's count below the bracket: one atomic
  unsigned long long b = below;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) b += __shfl_xor(b, d, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = b;
  __syncthreads();
  const uint32_t nl = min(lcount, (uint32_t)kBracketKeys);
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
    for (int w = 0; w < kBracketThreads / 64; ++w) t += red[w];
    atomicAdd(&st->below, t);
    gbase = nl ? atomicAdd(&st->count, nl) : 0u;
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nl; i += kBracketThreads) {
    const uint64_t pos = (uint64_t)gbase + i;
    if (pos < a.cap) a.compact[pos] = lbuf[i];
    else st->overflow = 1u;
  }
}

// The digit passes run over the bracket's compact copy if it was taken, did
// not overflow and holds the target rank; else over the tensor.  Every
// reader decides from the counters the bracket pass left, so no workgroup
// has to publish the decision.
__device__ __forceinline__ bool compact_hit(const SelectState *st) {
  const uint64_t k = st->rank0, b = st->below;
  return st->mode == 1u && !st->overflow && k >= b && k - b < st->count;
}

// The rank the first digit pass looks for: inside the compact copy, the
// keys below the bracket are already counted.
__device__ __forceinline__ uint64_t first_rank(const SelectState *st) {
  return compact_hit(st) ? st->rank0 - st->below : st->rank0;
}

// The digits of a selection: keys d = u - base whose low W bits vary, and
// per pass the digit's position and width (bits shift .. shift + width - 1
// of d; the widths add up to W, the last digit's shift is 0).  Every reader
// derives it from the bracket's counters, like compact_hit.
struct DigitPlan {
  uint32_t base;
  int shift[3], width[3];
};

__device__ __forceinline__ DigitPlan digit_plan(const SelectState *st) {
  DigitPlan p;
  uint32_t span = 0x7FFFFFFFu;  // the whole tensor: every key
  p.base = 0u;
  if (compact_hit(st)) {
    p.base = st->lo;
    span = st->hi - st->lo;
  }
  const int w = span ? 32 - __clz((int)span) : 0;
  p.shift[0] = max(w - 12, 0);
  p.width[0] = w - p.shift[0];
  p.shift[1] = max(p.shift[0] - 12, 0);
  p.width[1] = p.shift[0] - p.shift[1];
  p.shift[2] = 0;
  p.width[2] = p.shift[1];  // <= 8: w <= 32
  return p;
}

// Small tensors skip the bracket: the digit passes run over the tensor.
__global__ void select_full_kernel(SelectState *st, uint64_t rank) {
  st->mode = 0u;
  st->rank0 = rank;
}

template <int kPass>
__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(SelArgs a) {
  __shared__ uint32_t bins[kBins];
  for (int i = threadIdx.x; i < kBins; i += kSelThreads) bins[i] = 0u;
  __syncthreads();
  const DigitPlan pl = digit_plan(a.state);
  const int sh = pl.shift[kPass];
  const uint32_t mask = (1u << pl.width[kPass]) - 1u;
  // keys of this pass: the higher digits (d >> the previous digit's shift)
  // equal the prefix found so far
  const int psh = kPass == 0 ? 0 : pl.shift[kPass - 1];
  const uint32_t prefix = kPass == 0 ? 0u : a.state->prefix;
  auto count = [&](uint32_t u) {
    const uint32_t d = u - pl.base;
    if (kPass == 0 || (d >> psh) == prefix) atomicAdd(&bins[(d >> sh) & mask], 1u);
  };
  if (compact_hit(a.state)) {
    // The bracket's compact copy: keys already, all in [lo, hi].  Four keys
    // per 16-byte load and two loads in flight per thread (one at a time,
    // the loop waited out a load latency per key); then the last n % 4.
    const uint32_t n = a.state->count, n4 = n / 4;
    const uint4 *c4 = reinterpret_cast<const uint4 *>(a.compact);  // 256-byte aligned
    const uint32_t stride = gridDim.x * kSelThreads;
    for (uint32_t i = blockIdx.x * kSelThreads + threadIdx.x; i < n4; i += 2 * stride) {
      const bool two = i + stride < n4;
      const uint4 k0 = c4[i];
      const uint4 k1 = c4[two ? i + stride : i];
      count(k0.x);
      count(k0.y);
      count(k0.z);
      count(k0.w);
      if (two) {
        count(k1.x);
        count(k1.y);
        count(k1.z);
        count(k1.w);
      }
    }
    const uint32_t t = 4 * n4 + blockIdx.x * kSelThreads + threadIdx.x;
    if (t < n) count(a.compact[t]);
  } else {
    const uint64_t vpr = (uint64_t)(a.cols / 4);  // float4 per row
    const uint64_t nvec = (uint64_t)a.rows * vpr;
    for (uint64_t v = (uint64_t)blockIdx.x * kSelThreads + threadIdx.x; v < nvec;
         v += (uint64_t)gridDim.x * kSelThreads) {
      const float4 q = *reinterpret_cast<const float4 *>(a.x + vec_off(v, vpr, a.ld));
      count(abs_u(q.x));
      count(abs_u(q.y));
      count(abs_u(q.z));
      count(abs_u(q.w));
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kSelThreads)
    if (bins[i]) atomicAdd(&a.hist[i], bins[i]);
}

// One workgroup: find the bin holding the rank (0-based, ascending) among
// this pass's elements, narrow the prefix (d >> this digit's shift), and
// clear the histogram.  On the last pass the prefix is d itself: store the
// value base + d.
template <int kPass>
__global__ __launch_bounds__(kSelThreads) void select_scan_kernel(SelectState *st, uint32_t *hist) {
  __shared__ uint64_t part[kSelThreads];
  constexpr int kPer = kBins / kSelThreads;  // bins per thread
  const DigitPlan pl = digit_plan(st);
  const uint64_t rank = kPass == 0 ? first_rank(st) : st->rank;
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
    const uint32_t dg = (uint32_t)(threadIdx.x * kPer + b);
    const uint32_t prefix = kPass == 0 ? dg : ((st->prefix << pl.width[kPass]) | dg);
    st->prefix = prefix;
    st->rank = rank - below;
    if (kPass == 2) st->value = __uint_as_float(pl.base + prefix);
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

// Four elements of g at element offset off.
__device__ __forceinline__ float4 load4(const NormArgs &a, uint64_t off) {
  if (a.bf16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.g) + off);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xFFFF0000u));
  }
  return *reinterpret_cast<const float4 *>(static_cast<const float *>(a.g) + off);
}

__global__ __launch_bounds__(kSelThreads) void norm_partial_kernel(NormArgs a) {
  __shared__ double red[kSelThreads];
  const uint64_t vpr = (uint64_t)(a.cols / 4);
  const uint64_t nvec = (uint64_t)a.rows * vpr;
  double s = 0.0;
  for (uint64_t v = (uint64_t)blockIdx.x * kSelThreads + threadIdx.x; v < nvec;
       v += (uint64_t)gridDim.x * kSelThreads) {
    const float4 q = load4(a, vec_off(v, vpr, a.ld));
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
    const float4 q = load4(a, vec_off(v, vpr, a.ld));
    *reinterpret_cast<float4 *>(a.x + vec_off(v, vpr, a.xld)) = make_float4(q.x * inv, q.y * inv, q.z * inv, q.w * inv);
  }
}

int stride_grid(uint64_t nvec, uint64_t cap) {
  const uint64_t g = (nvec + kSelThreads - 1) / kSelThreads;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

nvfp4_status launch_abs_select(const float *x, int64_t rows, int64_t cols, int64_t ld, uint64_t rank,
                               SelectState *state, uint32_t *hist, uint32_t *compact, uint64_t cap,
                               hipStream_t s) {
  if (rows <= 0 || cols <= 0) return NVFP4_EINVAL;
  SelArgs a{x, rows, cols, ld, state, hist, compact, cap};
  const uint64_t n = (uint64_t)rows * (uint64_t)cols;
  const int g = stride_grid(n / 4, 2048);
  // With the bracket the digit passes read a few percent of the keys: fewer
  // workgroups (each clears and flushes a whole histogram); if the bracket
  // misses they cover the tensor with the same grid, only slower.
  int gh = g;
  if (n >= 32ull * kSamples && compact && cap > 0) {
    hipLaunchKernelGGL(select_sample_kernel, dim3(1), dim3(kSampleThreads), 0, s, a, rank);
    hipLaunchKernelGGL(select_bracket_kernel, dim3(256), dim3(kBracketThreads), 0, s, a);
    gh = g < 256 ? g : 256;
  } else {
    hipLaunchKernelGGL(select_full_kernel, dim3(1), dim3(1), 0, s, state, rank);
  }
  hipLaunchKernelGGL(select_hist_kernel<0>, dim3(gh), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_scan_kernel<0>, dim3(1), dim3(kSelThreads), 0, s, state, hist);
  hipLaunchKernelGGL(select_hist_kernel<1>, dim3(gh), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_scan_kernel<1>, dim3(1), dim3(kSelThreads), 0, s, state, hist);
  hipLaunchKernelGGL(select_hist_kernel<2>, dim3(gh), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_scan_kernel<2>, dim3(1), dim3(kSelThreads), 0, s, state, hist);
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
