// quantize.hip -- NVFP4 quantization kernels for gfx950.
//
// Two passes over HBM-resident input: an amax pass (per-tensor max |v| after
// the optional random Hadamard transform, reduced per wavefront and
// workgroup, one atomicMax per workgroup), then an encode pass that derives
// the tensor scale, the per-16 E4M3 block scales and the E2M1 codes.
// Quantization of the weights and activations that feed NVFP4 GEMMs is the
// step "NVIDIA acelera o pre-treinamento de LLM ..." describes in "Como o
// Treinamento Mixed-Precision Funciona com NVFP4"; the Hadamard mixing and
// stochastic rounding follow "Full-Stack FP4 ...", section 2.2.
//
// Row-wise ("along cols"): one lane owns half of a 16-element block (one
// 16-byte BF16 load); the two halves of a block sit in an even/odd lane pair
// and meet through a lane swap for the block maximum and the last Hadamard
// stage.  Consecutive lanes read consecutive 16-byte chunks.
// Transposing ("along rows"): one lane owns 8 input columns x 16 input rows,
// i.e. 8 complete blocks of the transposed view, so the transform and the
// block maximum stay in registers; consecutive lanes read consecutive
// 16-byte chunks of each row, and a lane walks 16 consecutive row blocks so
// its 8-byte code stores for a column fill whole 128-byte lines.
#include <hip/hip_runtime.h>

#include "device_codec.hpp"
#include "internal.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBlocksPerLane = 16;  // transposing kernel: 256 input rows per lane

struct RowArgs {
  const void *x;
  uint64_t half_blocks;  // batch * rows * cols / 8
  uint64_t hb_per_row;   // cols / 8
  int64_t rows, ld, bstride;
  uint8_t *codes, *scales;
  float *tensor_scale;
  QuantCtrl *ctrl;
  uint64_t sr_seed, rht_seed;
  uint32_t sr_stream;
};

struct ColArgs {
  const void *x;
  int64_t batch, R, C, ld, bstride;  // input [batch][R][C]; R % 16 == 0
  int64_t col_groups;                // ceil(C / 8)
  int64_t row_groups;                // ceil(R / 16 / kRowBlocksPerLane)
  uint64_t units;                    // batch * row_groups * col_groups
  bool vec_ok;                       // rows and batches start on 16-byte boundaries
  uint8_t *codes, *scales;
  float *tensor_scale;
  QuantCtrl *ctrl;
  uint64_t sr_seed, rht_seed;
  uint32_t sr_stream;
};

__device__ __forceinline__ uint32_t load_amax(const QuantCtrl *ctrl) {
  return __hip_atomic_load(&ctrl->amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup max -> one atomicMax per workgroup.
__device__ __forceinline__ void block_amax_commit(uint32_t m, QuantCtrl *ctrl) {
  __shared__ uint32_t part[kThreads / 64];
  m = wave_max_u32(m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = max(r, part[i]);
    atomicMax(&ctrl->amax_bits, r);
  }
}

// The last workgroup of the encode pass restores the control words to zero.
__device__ __forceinline__ void encode_finish(QuantCtrl *ctrl, float *tensor_scale, float st) {
  __syncthreads();
  if (threadIdx.x == 0) {
    if (blockIdx.x == 0) *tensor_scale = st;
    __threadfence();
    const uint32_t old = atomicAdd(&ctrl->done, 1u);
    if (old == gridDim.x - 1) {
      __hip_atomic_store(&ctrl->amax_bits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Per-block scale selection, shared by both layouts.
struct BlockScale {
  uint32_t code;  // E4M3 byte
  float recip;    // fl(1 / fl(E4M3(code) * s_t)), 0 for a zero scale
};

__device__ __forceinline__ BlockScale block_scale(float block_max, float st, float d6) {
  BlockScale b;
  b.code = (st > 0.0f) ? e4m3_encode(block_max / d6) : 0u;
  const float e = e4m3_value(b.code) * st;
  b.recip = (e == 0.0f) ? 0.0f : 1.0f / e;
  return b;
}

// ---------------------------------------------------------------------------
// Row-wise kernels
// ---------------------------------------------------------------------------

template <bool kBF16, bool kContig>
__device__ __forceinline__ void row_load(const RowArgs &a, uint64_t h, float (&v)[8]) {
  int64_t off;
  if (kContig) {
    off = (int64_t)(8 * h);
  } else {
    const uint64_t row = h / a.hb_per_row;
    const uint64_t hc = h - row * a.hb_per_row;
    const uint64_t b = row / (uint64_t)a.rows;
    const uint64_t r = row - b * (uint64_t)a.rows;
    off = (int64_t)b * a.bstride + (int64_t)r * a.ld + (int64_t)(8 * hc);
  }
  if (kBF16) {
    const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + off);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
    const float4 p = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + off);
    const float4 q = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + off + 4);
    v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w; v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
  }
}

template <bool kBF16, bool kRHT, bool kContig>
__global__ __launch_bounds__(kThreads) void row_amax_kernel(RowArgs a) {
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;
  uint32_t m = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t h = (uint64_t)blockIdx.x * kThreads + threadIdx.x; h < a.half_blocks; h += stride) {
    float v[8];
    row_load<kBF16, kContig>(a, h, v);
    if (kRHT) rht16_pair(v, mask, (h & 1) != 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max(m, abs_bits(v[j]));
  }
  block_amax_commit(m, a.ctrl);
}

template <bool kBF16, bool kRHT, bool kSR, bool kContig>
__global__ __launch_bounds__(kThreads) void row_encode_kernel(RowArgs a) {
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;
  const float amax = __uint_as_float(load_amax(a.ctrl));
  const float st = amax / 2688.0f;
  const float d6 = 6.0f * st;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t h = (uint64_t)blockIdx.x * kThreads + threadIdx.x; h < a.half_blocks; h += stride) {
    const bool odd = (h & 1) != 0;
    float v[8];
    row_load<kBF16, kContig>(a, h, v);
    if (kRHT) rht16_pair(v, mask, odd);
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max(m, abs_bits(v[j]));
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    const BlockScale bs = block_scale(__uint_as_float(m), st, d6);
    uint32_t packed = 0;
    if (kSR) {
      const u32x4 r = sr_block(h, a.sr_stream, a.sr_seed);
#pragma unroll
      for (int j = 0; j < 8; ++j) packed |= e2m1_sr(v[j] * bs.recip, sr_word(r, j)) << (4 * j);
    } else {
      float q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = v[j] * bs.recip;
      packed = e2m1_rne8(q);
    }
    *reinterpret_cast<uint32_t *>(a.codes + 4 * h) = packed;
    if (!odd) a.scales[h >> 1] = (uint8_t)bs.code;
  }
  encode_finish(a.ctrl, a.tensor_scale, st);
}

// ---------------------------------------------------------------------------
// Transposing kernels
// ---------------------------------------------------------------------------

// 16 rows x 8 columns of raw input held as BF16 pairs (4 dwords per row) or
// FP32 (8 floats per row).  Columns at or beyond C read as zero.
template <bool kBF16>
struct ColTile {
  uint32_t w[16][kBF16 ? 4 : 8];

  __device__ __forceinline__ float at(int row, int col) const {
    if (kBF16) return (col & 1) ? bf16_hi(w[row][col >> 1]) : bf16_lo(w[row][col >> 1]);
    return __uint_as_float(w[row][col]);
  }
};

template <bool kBF16>
__device__ __forceinline__ void col_load(const ColArgs &a, int64_t b, int64_t rb, int64_t cg,
                                         ColTile<kBF16> &t) {
  const int64_t c0 = 8 * cg;
  const bool full = a.vec_ok && c0 + 8 <= a.C;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t off = b * a.bstride + (16 * rb + j) * a.ld + c0;
    if (kBF16) {
      const uint16_t *p = static_cast<const uint16_t *>(a.x) + off;
      if (full) {
        const uint4 q = *reinterpret_cast<const uint4 *>(p);
        t.w[j][0] = q.x; t.w[j][1] = q.y; t.w[j][2] = q.z; t.w[j][3] = q.w;
      } else {
        uint32_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = (c0 + i < a.C) ? p[i] : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) t.w[j][i] = e[2 * i] | (e[2 * i + 1] << 16);
      }
    } else {
      const float *p = static_cast<const float *>(a.x) + off;
      if (full) {
        const float4 q0 = *reinterpret_cast<const float4 *>(p);
        const float4 q1 = *reinterpret_cast<const float4 *>(p + 4);
        t.w[j][0] = __float_as_uint(q0.x); t.w[j][1] = __float_as_uint(q0.y);
        t.w[j][2] = __float_as_uint(q0.z); t.w[j][3] = __float_as_uint(q0.w);
        t.w[j][4] = __float_as_uint(q1.x); t.w[j][5] = __float_as_uint(q1.y);
        t.w[j][6] = __float_as_uint(q1.z); t.w[j][7] = __float_as_uint(q1.w);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) t.w[j][i] = (c0 + i < a.C) ? __float_as_uint(p[i]) : 0u;
      }
    }
  }
}

__device__ __forceinline__ void col_unit(const ColArgs &a, uint64_t u, int64_t &b, int64_t &rbg,
                                         int64_t &cg) {
  cg = (int64_t)(u % (uint64_t)a.col_groups);
  const uint64_t t = u / (uint64_t)a.col_groups;
  rbg = (int64_t)(t % (uint64_t)a.row_groups);
  b = (int64_t)(t / (uint64_t)a.row_groups);
}

template <bool kBF16, bool kRHT>
__global__ __launch_bounds__(kThreads) void col_amax_kernel(ColArgs a) {
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;
  const int64_t RB = a.R / 16;
  uint32_t m = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t u = (uint64_t)blockIdx.x * kThreads + threadIdx.x; u < a.units; u += stride) {
    int64_t b, rbg, cg;
    col_unit(a, u, b, rbg, cg);
    const int64_t rb_end = min(RB, (rbg + 1) * kRowBlocksPerLane);
    for (int64_t rb = rbg * kRowBlocksPerLane; rb < rb_end; ++rb) {
      ColTile<kBF16> t;
      col_load<kBF16>(a, b, rb, cg, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = t.at(j, e);
        if (kRHT) rht16(v, mask);
#pragma unroll
        for (int j = 0; j < 16; ++j) m = max(m, abs_bits(v[j]));
      }
    }
  }
  block_amax_commit(m, a.ctrl);
}

template <bool kBF16, bool kRHT, bool kSR>
__global__ __launch_bounds__(kThreads) void col_encode_kernel(ColArgs a) {
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;
  const float amax = __uint_as_float(load_amax(a.ctrl));
  const float st = amax / 2688.0f;
  const float d6 = 6.0f * st;
  const int64_t RB = a.R / 16;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t u = (uint64_t)blockIdx.x * kThreads + threadIdx.x; u < a.units; u += stride) {
    int64_t b, rbg, cg;
    col_unit(a, u, b, rbg, cg);
    const int64_t rb_end = min(RB, (rbg + 1) * kRowBlocksPerLane);
    for (int64_t rb = rbg * kRowBlocksPerLane; rb < rb_end; ++rb) {
      ColTile<kBF16> t;
      col_load<kBF16>(a, b, rb, cg, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t c = 8 * cg + e;  // row of the transposed view
        if (c >= a.C) break;
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = t.at(j, e);
        if (kRHT) rht16(v, mask);
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) m = max(m, abs_bits(v[j]));
        const BlockScale bs = block_scale(__uint_as_float(m), st, d6);
        const int64_t vrow = b * a.C + c;  // row index in the [batch*C][R] view
        uint32_t lo = 0, hi = 0;
        if (kSR) {
          const uint64_t g0 = (uint64_t)(vrow * a.R + 16 * rb) / 8;
          const u32x4 r0 = sr_block(g0, a.sr_stream, a.sr_seed);
          const u32x4 r1 = sr_block(g0 + 1, a.sr_stream, a.sr_seed);
#pragma unroll
          for (int j = 0; j < 8; ++j) lo |= e2m1_sr(v[j] * bs.recip, sr_word(r0, j)) << (4 * j);
#pragma unroll
          for (int j = 0; j < 8; ++j) hi |= e2m1_sr(v[8 + j] * bs.recip, sr_word(r1, j)) << (4 * j);
        } else {
          float q[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) q[j] = v[j] * bs.recip;
          lo = e2m1_rne8(q);
          hi = e2m1_rne8(q + 8);
        }
        *reinterpret_cast<uint2 *>(a.codes + vrow * (a.R / 2) + 8 * rb) = make_uint2(lo, hi);
        a.scales[vrow * RB + rb] = (uint8_t)bs.code;
      }
    }
  }
  encode_finish(a.ctrl, a.tensor_scale, st);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

int grid_for(uint64_t items) {
  const uint64_t want = (items + kThreads - 1) / kThreads;
  const uint64_t cap = 256ull * 8;  // 8 workgroups per CU on a 256-CU part
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

template <bool kBF16, bool kRHT, bool kSR, bool kContig>
hipError_t run_row(const RowArgs &a, hipStream_t s) {
  const int g = grid_for(a.half_blocks);
  hipLaunchKernelGGL((row_amax_kernel<kBF16, kRHT, kContig>), dim3(g), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((row_encode_kernel<kBF16, kRHT, kSR, kContig>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool kBF16, bool kRHT, bool kSR>
hipError_t run_col(const ColArgs &a, hipStream_t s) {
  const int g = grid_for(a.units);
  hipLaunchKernelGGL((col_amax_kernel<kBF16, kRHT>), dim3(g), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((col_encode_kernel<kBF16, kRHT, kSR>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool kBF16, bool kRHT, bool kSR>
hipError_t dispatch_row(const RowArgs &a, bool contig, hipStream_t s) {
  return contig ? run_row<kBF16, kRHT, kSR, true>(a, s) : run_row<kBF16, kRHT, kSR, false>(a, s);
}

template <bool kBF16>
hipError_t dispatch_flags_row(const RowArgs &a, bool rht, bool sr, bool contig, hipStream_t s) {
  if (rht) return sr ? dispatch_row<kBF16, true, true>(a, contig, s) : dispatch_row<kBF16, true, false>(a, contig, s);
  return sr ? dispatch_row<kBF16, false, true>(a, contig, s) : dispatch_row<kBF16, false, false>(a, contig, s);
}

template <bool kBF16>
hipError_t dispatch_flags_col(const ColArgs &a, bool rht, bool sr, hipStream_t s) {
  if (rht) return sr ? run_col<kBF16, true, true>(a, s) : run_col<kBF16, true, false>(a, s);
  return sr ? run_col<kBF16, false, true>(a, s) : run_col<kBF16, false, false>(a, s);
}

__global__ void store_zero_scale(float *p) { *p = 0.0f; }

}  // namespace

nvfp4_status launch_quantize(const QuantProblem &p, hipStream_t s) {
  const int64_t qr = p.along_rows ? p.cols : p.rows;
  const int64_t qc = p.along_rows ? p.rows : p.cols;
  if (p.batch == 0 || qr == 0 || qc == 0) {
    hipLaunchKernelGGL(store_zero_scale, dim3(1), dim3(1), 0, s, p.tensor_scale);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
  }
  hipError_t err;
  if (!p.along_rows) {
    RowArgs a{};
    a.x = p.x;
    a.half_blocks = (uint64_t)(p.batch * p.rows * p.cols / 8);
    a.hb_per_row = (uint64_t)(p.cols / 8);
    a.rows = p.rows;
    a.ld = p.ld;
    a.bstride = p.bstride;
    a.codes = p.codes;
    a.scales = p.scales;
    a.tensor_scale = p.tensor_scale;
    a.ctrl = p.ctrl;
    a.sr_seed = p.sr_seed;
    a.rht_seed = p.rht_seed;
    a.sr_stream = p.sr_stream;
    const bool contig = (p.ld == p.cols) && (p.batch == 1 || p.bstride == p.rows * p.ld);
    err = p.bf16 ? dispatch_flags_row<true>(a, p.rht, p.sr, contig, s)
                 : dispatch_flags_row<false>(a, p.rht, p.sr, contig, s);
  } else {
    ColArgs a{};
    a.x = p.x;
    a.batch = p.batch;
    a.R = p.rows;
    a.C = p.cols;
    a.ld = p.ld;
    a.bstride = p.bstride;
    a.col_groups = (p.cols + 7) / 8;
    a.row_groups = (p.rows / 16 + kRowBlocksPerLane - 1) / kRowBlocksPerLane;
    a.units = (uint64_t)(a.batch * a.row_groups * a.col_groups);
    {
      const int64_t esize = p.bf16 ? 2 : 4;
      a.vec_ok = reinterpret_cast<uintptr_t>(p.x) % 16 == 0 && (p.ld * esize) % 16 == 0 &&
                 (p.batch == 1 || (p.bstride * esize) % 16 == 0);
    }
    a.codes = p.codes;
    a.scales = p.scales;
    a.tensor_scale = p.tensor_scale;
    a.ctrl = p.ctrl;
    a.sr_seed = p.sr_seed;
    a.rht_seed = p.rht_seed;
    a.sr_stream = p.sr_stream;
    err = p.bf16 ? dispatch_flags_col<true>(a, p.rht, p.sr, s) : dispatch_flags_col<false>(a, p.rht, p.sr, s);
  }
  return err == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace nvfp4
