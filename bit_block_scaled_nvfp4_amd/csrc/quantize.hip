// quantize.hip -- NVFP4 quantization kernels for gfx950.
//
// Quantization of the weights and activations that feed NVFP4 GEMMs is the
// step "NVIDIA acelera o pre-treinamento de LLM ..." describes in "Como o
// Treinamento Mixed-Precision Funciona com NVFP4"; the Hadamard mixing and
// stochastic rounding follow "Full-Stack FP4 ...", section 2.2.  Every block
// scale depends on the per-tensor amax, so the tensor is either read once and
// held on chip across a grid-wide barrier, or read twice.
//
// Row-wise ("along cols", blocks along the contiguous dimension), one lane
// owns one whole 16-element block (two 16-byte BF16 loads), so the transform,
// the block maximum and the block scale stay in the lane.
//  * Single pass (tensors that fit in the register files): a grid of one
//    1024-thread workgroup per CU loads every lane's blocks (up to 9 per
//    lane for BF16, 37.7M elements on 256 CUs) into registers, every load
//    issued before the first wait, reduces the amax per wavefront and
//    workgroup, meets the rest of the grid at an epoch barrier, then encodes
//    from registers.  HBM sees one read of the input and one write of codes
//    and scales.  Up to four tensors (a GEMM's operands) share one launch.
//  * Two passes (larger tensors or strided rows): an amax kernel and an
//    encode kernel over the same block order; the second read largely hits
//    the 256 MB Infinity Cache for tensors that fit it.
// Transposing ("along rows"): one lane owns 8 input columns x 16 input rows,
// i.e. 8 complete blocks of the transposed view, so the transform and the
// block maximum stay in the lane, and codes are staged in LDS so each
// transposed row's code line is written by one workgroup.
//  * Single pass (BF16, grids of at most one workgroup per CU): 512- or
//    1024-row x 128-column tiles held in registers across the same barrier.
//  * Two passes otherwise: 256-row x 128-column tiles.
//
// Encode of a block: S = E4M3(fl(max|v| / fl(6 s_t))), q = fl(v * r_S) with
// r_S = fl(1 / fl(E4M3(S) * s_t)) from a 127-entry LDS table built once per
// workgroup, then E2M1 (the hardware converters: round to nearest even, or
// stochastic rounding driven by the element's Philox word).
#include <hip/hip_runtime.h>

#include <atomic>

#include "device_codec.hpp"
#include "internal.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;           // two-pass kernels
constexpr int kFusedThreads = 1024;     // single-pass kernel, one workgroup per CU
constexpr int kBatch = 4;               // two-pass row kernels: blocks loaded per lane before use
constexpr uint32_t kSpinLimit = 1u << 22;  // polls before a barrier wait gives up (~1 s)

template <bool kBF16, bool kRHT, bool kSR>
struct Fused {
  // Blocks held per lane: 37.7M BF16 (16.8M FP32) elements on 256 CUs, the
  // most that fits the 128-VGPR budget of 1024-thread workgroups without
  // spilling (BF16 with both the transform and stochastic rounding: 29.4M).
  static constexpr int kMaxBlocks = kBF16 ? (kRHT && kSR ? 7 : 9) : 4;
};

// ---------------------------------------------------------------------------
// Shared pieces
// ---------------------------------------------------------------------------

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));

// Streaming 16-byte load / 8-byte store that bypass cache allocation: the
// input is read exactly once and the codes are not read back here.
__device__ __forceinline__ uint4 ld_stream(const void *p) {
  const u32x4v v = __builtin_nontemporal_load(static_cast<const u32x4v *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void *p, uint2 v) {
  const u32x2v t = {v.x, v.y};
  __builtin_nontemporal_store(t, static_cast<u32x2v *>(p));
}

// 16 raw input elements of one block: BF16 pairs in 8 dwords or FP32 in 16.
template <bool kBF16>
struct RawBlock {
  uint32_t w[kBF16 ? 8 : 16];
  template <bool kStream = true>
  __device__ __forceinline__ void load(const void *x, int64_t off) {
    const uint8_t *p = static_cast<const uint8_t *>(x) + off * (kBF16 ? 2 : 4);
#pragma unroll
    for (int i = 0; i < (kBF16 ? 2 : 4); ++i) {
      const uint4 a = kStream ? ld_stream(p + 16 * i) : *reinterpret_cast<const uint4 *>(p + 16 * i);
      w[4 * i] = a.x; w[4 * i + 1] = a.y; w[4 * i + 2] = a.z; w[4 * i + 3] = a.w;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < (kBF16 ? 8 : 16); ++i) w[i] = 0u;
  }
  // Hide the words from value numbering so that a later unpack is redone
  // rather than kept alive in 16 extra registers per block.
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int i = 0; i < (kBF16 ? 8 : 16); ++i) asm volatile("" : "+v"(w[i]));
  }
  // max |v| over the block as FP32 bits, straight from BF16 words: |x|
  // orders like the unsigned 15-bit magnitude field, so packed 16-bit maxima
  // of (w & 0x7FFF7FFF) give the largest magnitude, whose FP32 bits are its
  // BF16 bits shifted left by 16.  Equal to max_abs16 of the unpacked values.
  __device__ __forceinline__ uint32_t max_abs_bf16() const {
    static_assert(kBF16, "BF16 blocks only");
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    return (uint32_t)(m.x > m.y ? m.x : m.y) << 16;
  }
  __device__ __forceinline__ void values(float (&v)[16]) const {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      v[j] = kBF16 ? ((j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1])) : __uint_as_float(w[j]);
  }
};

// max |v| over 16 values as FP32 bits.
__device__ __forceinline__ uint32_t max_abs16(const float (&v)[16]) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = max(m, abs_bits(v[j]));
  return m;
}

// Block scale code from the block maximum (RNE E4M3, S = 0 when s_t = 0).
__device__ __forceinline__ uint32_t block_scale_code(uint32_t bmax_bits, float st, float d6) {
  return (st > 0.0f) ? e4m3_encode(__uint_as_float(bmax_bits) / d6) : 0u;
}

// recip[S] = fl(1 / fl(E4M3(S) * s_t)), or 0 when that product is 0.
__device__ __forceinline__ void build_recip_table(float *recip, float st) {
  for (int s = threadIdx.x; s < 127; s += blockDim.x) {
    const float e = e4m3_value((uint32_t)s) * st;
    recip[s] = (e == 0.0f) ? 0.0f : 1.0f / e;
  }
}

// Encode 16 values (logical element index n0 of the first) with multiplier r
// into two dwords of codes.
template <bool kSR>
__device__ __forceinline__ uint2 encode16(const float (&v)[16], float r, uint64_t n0, uint32_t stream,
                                          uint64_t seed) {
  float q[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) q[j] = v[j] * r;
  if (kSR) {
    const u32x4 r0 = sr_block(n0 / 8, stream, seed);
    const u32x4 r1 = sr_block(n0 / 8 + 1, stream, seed);
    return make_uint2(e2m1_sr8(q, r0.x, r0.y, r0.z, r0.w), e2m1_sr8(q + 8, r1.x, r1.y, r1.z, r1.w));
  }
  return make_uint2(e2m1_rne8(q), e2m1_rne8(q + 8));
}

// Device-scope relaxed atomics: performed at the memory-side coherence
// point, with no cache writeback or invalidation around them.
template <typename T>
__device__ __forceinline__ T atomic_load_dev(const T *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void atomic_store_dev(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Stall until a returning atomic has completed (its value is consumed).
template <typename T>
__device__ __forceinline__ void wait_for(T v) {
  asm volatile("" ::"v"(v));
}

// Two-pass tensor max as FP32 bits: the max of the eight partial slots.
__device__ __forceinline__ uint32_t load_amax(const QuantCtrl *ctrl) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, atomic_load_dev(&ctrl->part[i].v));
  return m;
}

// Workgroups per barrier slot (slot = blockIdx mod 8) and slots in use, for
// the launch's own grid size.
__device__ __forceinline__ unsigned slots_in_use() { return min(gridDim.x, 8u); }
__device__ __forceinline__ unsigned per_slot(int slot) {
  return gridDim.x / 8 + ((unsigned)slot < gridDim.x % 8 ? 1u : 0u);
}

// Single-pass grid barrier, thread 0 of each workgroup: arrive at epoch e and
// wait for its release.  The last arrival at a slot stores the slot's counter
// back to zero and bumps `top`; the last of those stores `top` back to zero
// and publishes e + 1.  Nothing else touches these counters until the kernel
// ends, so the next call (ordered after this one on its stream) starts from
// zero whatever its grid size.  All control words are device-scope atomics at
// the coherence point, so relaxed ordering plus the caller's explicit
// completion waits suffice (acquire/release would flush and invalidate the L2
// on every poll).  The wait is bounded: on expiry the sticky timeout word is
// set (completed before the workgroup goes on) and true is returned; the
// kernel still finishes, and its last workgroup then writes a NaN tensor
// scale.
__device__ __forceinline__ bool fused_arrive_wait(QuantCtrl *ctrl, unsigned long long e, int slot) {
  const unsigned long long old =
      __hip_atomic_fetch_add(&ctrl->arrive[slot].v, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1 == per_slot(slot)) {
    atomic_store_dev(&ctrl->arrive[slot].v, 0ull);
    const unsigned long long t = __hip_atomic_fetch_add(&ctrl->top.v, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t + 1 == slots_in_use()) {
      atomic_store_dev(&ctrl->top.v, 0ull);
      atomic_store_dev(&ctrl->release.v, e + 1);
    }
  }
  const uint32_t lim = atomic_load_dev(&ctrl->spin_limit);
  const uint32_t limit = lim ? lim : kSpinLimit;
  for (uint32_t spin = 0;; ++spin) {
    if (atomic_load_dev(&ctrl->release.v) > e) return false;
    if (spin >= limit) {
      wait_for(__hip_atomic_fetch_or(&ctrl->timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Thread 0 of each workgroup at the end of a single-pass kernel: true for the
// last workgroup of the grid to get here (counted like the barrier's
// arrivals, in the `fin` words, each restored to zero by its last arrival).
// Every workgroup has passed or given up its barrier wait before it counts,
// and a workgroup that gave up set the timeout word before that, so the last
// one sees every expiry of the call.
__device__ __forceinline__ bool fused_last_to_finish(QuantCtrl *ctrl, int slot) {
  const uint32_t old = __hip_atomic_fetch_add(&ctrl->arrive[slot].fin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1 != per_slot(slot)) return false;
  atomic_store_dev(&ctrl->arrive[slot].fin, 0u);
  const uint32_t t = __hip_atomic_fetch_add(&ctrl->top.fin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t + 1 != slots_in_use()) return false;
  atomic_store_dev(&ctrl->top.fin, 0u);
  return true;
}

// The tensor scale a single-pass call publishes: s_t, or NaN once any barrier
// wait on this workspace has expired (the codes are then unreliable).
__device__ __forceinline__ float published_scale(const QuantCtrl *ctrl, float st) {
  return atomic_load_dev(&ctrl->timeout) != 0u ? __builtin_nanf("") : st;
}

// Workgroup max -> one atomicMax per workgroup into slot blockIdx mod 8
// (two-pass amax kernels).
__device__ __forceinline__ void block_amax_commit(uint32_t m, QuantCtrl *ctrl) {
  __shared__ uint32_t part[16];
  m = wave_max_u32(m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = max(r, part[i]);
    __hip_atomic_fetch_max(&ctrl->part[blockIdx.x & 7].v, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The last workgroup of an encode pass restores the two-pass words to zero.
__device__ __forceinline__ void encode_finish(QuantCtrl *ctrl, float *tensor_scale, float st) {
  __syncthreads();
  if (threadIdx.x == 0) {
    if (blockIdx.x == 0) *tensor_scale = st;
    // Every workgroup read the amax before arriving here; the last one to
    // arrive (seen through the returned count) clears the two-pass words.
    const uint32_t old = __hip_atomic_fetch_add(&ctrl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      for (int i = 0; i < 8; ++i) atomic_store_dev(&ctrl->part[i].v, 0u);
      atomic_store_dev(&ctrl->done, 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// Row-wise kernels
// ---------------------------------------------------------------------------

struct RowArgs {
  const void *x;
  uint64_t nblocks;   // batch * rows * cols / 16
  uint64_t bpr;       // blocks per row (cols / 16)
  int64_t rows, ld, bstride;
  uint8_t *codes, *scales;
  float *tensor_scale;
  QuantCtrl *ctrl;
  uint64_t sr_seed, rht_seed;
  uint32_t sr_stream;
  uint16_t *means;    // second-moment pre-step only: BF16 block means, one per block
  const float *clip;  // FP32 only: values are first clamped to [-*clip, *clip]
};

// x clamped to [-c, c]; NaN stays NaN.
__device__ __forceinline__ float clamp_abs(float x, float c) { return x > c ? c : (x < -c ? -c : x); }

// Second-moment pre-step of the quantized-state optimizer ("Full-Stack FP4
// ...", section 2.2: square root, tile mean, then the Hadamard transform) on
// one 16-element block of FP32 values: s_j = sqrt(v_j) (correctly rounded),
// the block mean mu = BF16_RNE(fl(sum_j s_j) / 16) with the sum taken left to
// right, and the residuals r_j = fl(s_j - mu) in place.  Returns mu's BF16
// bits.
__device__ __forceinline__ uint32_t sqrt_demean16(float (&v)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __builtin_sqrtf(v[j]);
  float sum = v[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) sum = sum + v[j];
  const uint32_t mb = pack_bf16x2_rne(sum * 0.0625f, 0.0f) & 0xFFFFu;  // the division by 16 is exact
  const float mu = __uint_as_float(mb << 16);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = v[j] - mu;
  return mb;
}

// Single pass: up to kMaxJobs contiguous tensors in one launch, each with
// its own tensor scale.  Global segment g belongs to the job whose
// [seg_begin, next seg_begin) range holds it.
constexpr int kMaxJobs = 4;
static_assert(kMaxJobs == kMaxGroup, "the group API and the kernel table hold the same number of jobs");
struct RowJob {
  const void *x;
  uint64_t nblocks;
  uint64_t seg_begin;
  uint8_t *codes, *scales;
  float *tensor_scale;
  QuantCtrl::Slot (*amax)[8];  // [2][8]: per epoch parity, per workgroup-index slot
};
struct FusedArgs {
  RowJob job[kMaxJobs];
  int njobs;
  uint64_t nseg;     // segments over all jobs
  QuantCtrl *ctrl;   // barrier counters
  uint64_t sr_seed, rht_seed;
  uint32_t sr_stream;
  uint32_t nseg_iters;  // segments per wavefront
};

// Element offset of block `blk` (row-major over [batch*rows][cols/16]).
template <bool kContig>
__device__ __forceinline__ int64_t row_block_offset(const RowArgs &a, uint64_t blk) {
  if (kContig) return (int64_t)(16 * blk);
  const uint64_t row = blk / a.bpr;
  const uint64_t cb = blk - row * a.bpr;
  const uint64_t b = row / (uint64_t)a.rows;
  const uint64_t r = row - b * (uint64_t)a.rows;
  return (int64_t)b * a.bstride + (int64_t)r * a.ld + (int64_t)(16 * cb);
}

// Wavefront segments: 64 consecutive blocks handled by one wavefront.  For a
// contiguous BF16 tensor the segment (2 KB) is read with two fully coalesced
// 16-byte loads per lane (chunks lane and 64 + lane), after which each even /
// odd lane pair swaps one half so that even lane 2k owns block 64 seg + k and
// odd lane 2k+1 owns block 64 seg + 32 + k.  Otherwise lane l owns block
// 64 seg + l and loads it directly.
//
// Loading is split in two so that a wavefront can have all of its segments'
// loads in flight before it waits for the first: issue_* only computes
// addresses and issues loads, finish_* (after the data arrived) does the lane
// exchange and returns the lane's block index.  Out-of-range chunks and
// blocks are not branched around (a branch whose other side writes the same
// registers makes the compiler wait for each load in turn): their indices
// are clamped to the last valid one, and the caller ignores blocks whose
// index is past the end.  kStream: non-temporal loads (data read once); the
// two-pass amax kernel uses cached loads instead so the encode pass can
// re-read from the Infinity Cache.
struct SegChunks {
  uint4 c0, c1;
};

template <bool kStream, typename Idx>
__device__ __forceinline__ SegChunks issue_segment_bf16(const void *x, Idx nchunks, Idx seg, int lane) {
  const uint4 *p = static_cast<const uint4 *>(x);
  const Idx last = nchunks - 1;
  const Idx c0 = seg * 128 + (Idx)lane, c1 = c0 + 64;
  const uint4 *p0 = p + (c0 < last ? c0 : last), *p1 = p + (c1 < last ? c1 : last);
  SegChunks r;
  r.c0 = kStream ? ld_stream(p0) : *p0;
  r.c1 = kStream ? ld_stream(p1) : *p1;
  return r;
}

template <typename Idx>
__device__ __forceinline__ Idx finish_segment_bf16(const SegChunks &s, Idx seg, int lane, RawBlock<true> &raw) {
  const bool odd = lane & 1;
  const uint4 send = odd ? s.c0 : s.c1;
  const uint4 recv = make_uint4(lane_xor1(send.x), lane_xor1(send.y), lane_xor1(send.z), lane_xor1(send.w));
  const uint4 lo = odd ? recv : s.c0, hi = odd ? s.c1 : recv;
  raw.w[0] = lo.x; raw.w[1] = lo.y; raw.w[2] = lo.z; raw.w[3] = lo.w;
  raw.w[4] = hi.x; raw.w[5] = hi.y; raw.w[6] = hi.z; raw.w[7] = hi.w;
  return seg * 64 + (Idx)((lane & 1) * 32 + (lane >> 1));
}

// Segment of any other layout (FP32, or rows with a stride): lane l loads
// block 64 seg + l whole, clamped to the last block.
template <bool kBF16, bool kContig, bool kStream>
__device__ __forceinline__ uint64_t issue_segment_direct(const RowArgs &a, uint64_t seg, int lane,
                                                         RawBlock<kBF16> &raw) {
  const uint64_t blk = seg * 64 + lane;
  raw.template load<kStream>(a.x, row_block_offset<kContig>(a, blk < a.nblocks ? blk : a.nblocks - 1));
  return blk;
}

// Segments of the two-pass row kernels: raw[i] and the block index of
// segment s0 + i * stride, all loads issued before any is waited for.
template <bool kBF16, bool kContig, bool kStream, int kN>
__device__ __forceinline__ void load_segments(const RowArgs &a, uint64_t s0, uint64_t stride, int lane,
                                              RawBlock<kBF16> (&raw)[kN], uint64_t (&blk)[kN]) {
  if constexpr (kBF16 && kContig) {
    SegChunks ch[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i) ch[i] = issue_segment_bf16<kStream, uint64_t>(a.x, 2 * a.nblocks, s0 + i * stride, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first exchange
#pragma unroll
    for (int i = 0; i < kN; ++i) blk[i] = finish_segment_bf16<uint64_t>(ch[i], s0 + i * stride, lane, raw[i]);
  } else {
#pragma unroll
    for (int i = 0; i < kN; ++i) blk[i] = issue_segment_direct<kBF16, kContig, kStream>(a, s0 + i * stride, lane, raw[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Encode one block (values already transformed) and store codes + scale.
template <bool kSR>
__device__ __forceinline__ void row_store_block(const RowArgs &a, uint64_t blk, const float (&v)[16], uint32_t S,
                                                const float *recip) {
  const uint2 c = encode16<kSR>(v, recip[S], 16 * blk, a.sr_stream, a.sr_seed);
  st_stream(a.codes + 8 * blk, c);
  a.scales[blk] = (uint8_t)S;
}

template <bool kBF16, bool kRHT, bool kSR>
__global__ __launch_bounds__(kFusedThreads, kFusedThreads / 256) void row_fused_kernel(FusedArgs a) {
  constexpr int kMax = Fused<kBF16, kRHT, kSR>::kMaxBlocks;
  constexpr int kWaves = kFusedThreads / 64;
  __shared__ float recip[kMaxJobs][128];
  __shared__ uint32_t part[kWaves][kMaxJobs];
  __shared__ unsigned long long s_epoch;
  __shared__ float s_st[kMaxJobs];
  QuantCtrl *ctrl = a.ctrl;
  const int slot = blockIdx.x & 7;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int njobs = a.njobs;

  // The epoch (completed single-pass calls on this workspace) cannot advance
  // before this workgroup arrives, so reading it here is race free.
  if (threadIdx.x == 0) s_epoch = atomic_load_dev(&ctrl->release.v);

  // 32-bit indices throughout: the launcher only runs this kernel within its
  // capacity (at most kMax segments per wavefront of one grid).
  const uint32_t nwaves = gridDim.x * kWaves;
  const uint32_t gwave = blockIdx.x * kWaves + wave;
  const uint32_t nseg = (uint32_t)a.nseg;
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;

  // Phase 1: every segment's loads are issued before the first is waited
  // for, then the block maxima.  A segment belongs to one job, so the job
  // index is uniform across the wavefront.  Iterations at or past nseg_iters
  // (uniform over the grid) load nothing; within them, a segment past the
  // end of the last job loads that job's final chunk again (clamped, in
  // bounds) and is marked invalid.
  RawBlock<kBF16> raw[kMax];
  uint32_t blk[kMax];
  int jb[kMax];
  uint32_t bmax[kMax];
  {
    uint32_t seg[kMax];
    const void *xs[kMax];
#pragma unroll
    for (int it = 0; it < kMax; ++it) {
      const uint32_t g = it * nwaves + gwave;
      const int j = (njobs > 1 && g >= (uint32_t)a.job[1].seg_begin) + (njobs > 2 && g >= (uint32_t)a.job[2].seg_begin) +
                    (njobs > 3 && g >= (uint32_t)a.job[3].seg_begin);
      jb[it] = j;
      xs[it] = j == 0 ? a.job[0].x : j == 1 ? a.job[1].x : j == 2 ? a.job[2].x : a.job[3].x;
      const uint32_t sb = (uint32_t)(j == 0 ? a.job[0].seg_begin : j == 1 ? a.job[1].seg_begin
                                     : j == 2 ? a.job[2].seg_begin : a.job[3].seg_begin);
      seg[it] = g - sb;
    }
    auto job_nblocks = [&](int j) -> uint32_t {
      return (uint32_t)(j == 0 ? a.job[0].nblocks : j == 1 ? a.job[1].nblocks : j == 2 ? a.job[2].nblocks
                                                                                       : a.job[3].nblocks);
    };
    if constexpr (kBF16) {
      SegChunks ch[kMax];
#pragma unroll
      for (int it = 0; it < kMax; ++it)
        if (it < (int)a.nseg_iters)
          ch[it] = issue_segment_bf16<true, uint32_t>(xs[it], 2 * job_nblocks(jb[it]), seg[it], lane);
#pragma unroll
      for (int it = 0; it < kMax; ++it) {
        if (it < (int)a.nseg_iters) blk[it] = finish_segment_bf16<uint32_t>(ch[it], seg[it], lane, raw[it]);
        else raw[it].zero();
      }
    } else {
#pragma unroll
      for (int it = 0; it < kMax; ++it) {
        const uint32_t nb = job_nblocks(jb[it]);
        blk[it] = seg[it] * 64 + lane;
        if (it < (int)a.nseg_iters) raw[it].load(xs[it], (int64_t)16 * (blk[it] < nb ? blk[it] : nb - 1));
        else raw[it].zero();
      }
    }
#pragma unroll
    for (int it = 0; it < kMax; ++it) {
      const uint32_t g = it * nwaves + gwave;
      if (!(it < (int)a.nseg_iters && g < nseg) || blk[it] >= job_nblocks(jb[it])) blk[it] = ~0u;
    }
  }
  uint32_t mj[kMaxJobs] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int it = 0; it < kMax; ++it) {
    if constexpr (kBF16 && !kRHT) {
      bmax[it] = raw[it].max_abs_bf16();
    } else {
      float v[16];
      raw[it].values(v);
      if (kRHT) {
        rht16_unscaled(v, mask);
        bmax[it] = quarter_max_bits(max_abs16(v));
      } else {
        bmax[it] = max_abs16(v);
      }
    }
    if (blk[it] == ~0u) bmax[it] = 0u;
#pragma unroll
    for (int j = 0; j < kMaxJobs; ++j)
      if (jb[it] == j) mj[j] = max(mj[j], bmax[it]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < kMaxJobs; ++j) {
    if (j < njobs) {
      const uint32_t m = wave_max_u32(mj[j]);
      if (lane == 0) part[wave][j] = m;
    }
  }
  __syncthreads();

  // Grid barrier: publish the workgroup maxima, arrive, wait for the epoch
  // to complete, then read the tensor maxima.  All control words are
  // device-scope atomics at the coherence point, so relaxed ordering plus
  // explicit completion waits suffice (acquire/release would flush and
  // invalidate the L2 on every poll).  The wait is bounded; on expiry the
  // timeout word is set and the kernel still finishes.
  if (threadIdx.x == 0) {
    const unsigned long long e = s_epoch;
    // Slots of the next epoch are unused since the call before this one
    // ended.  Every table entry that has slots is cleared, not only this
    // call's jobs: a later call on the workspace may have more jobs.
    if (blockIdx.x == 0) {
      for (int j = 0; j < kMaxJobs; ++j) {
        if (a.job[j].amax == nullptr) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) atomic_store_dev(&a.job[j].amax[(e + 1) & 1][i].v, 0u);
      }
    }
    for (int j = 0; j < njobs; ++j) {
      uint32_t wm = part[0][j];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) wm = max(wm, part[w][j]);
      const uint32_t prev = __hip_atomic_fetch_max(&a.job[j].amax[e & 1][slot].v, wm, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      wait_for(prev);  // the max is performed before this workgroup counts as arrived
    }
    (void)fused_arrive_wait(ctrl, e, slot);
    for (int j = 0; j < njobs; ++j) {
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = max(am, atomic_load_dev(&a.job[j].amax[e & 1][i].v));
      s_st[j] = __uint_as_float(am) / 2688.0f;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < njobs * 128; t += kFusedThreads) {
    const int j = t >> 7, sc = t & 127;
    if (sc < 127) {
      const float e = e4m3_value((uint32_t)sc) * s_st[j];
      recip[j][sc] = (e == 0.0f) ? 0.0f : 1.0f / e;
    }
  }
  __syncthreads();

  // Phase 2: encode from registers.
#pragma unroll
  for (int it = 0; it < kMax; ++it) raw[it].opaque();
#pragma unroll
  for (int it = 0; it < kMax; ++it) {
    const int j = jb[it];
    if (blk[it] < (uint32_t)a.job[j].nblocks) {
      const float st = s_st[j];
      const uint32_t S = block_scale_code(bmax[it], st, 6.0f * st);
      float v[16];
      raw[it].values(v);
      if (kRHT) rht16(v, mask);
      const uint2 c = encode16<kSR>(v, recip[j][S], (uint64_t)16 * blk[it], a.sr_stream, a.sr_seed);
      // Uniform base plus a 32-bit lane offset (the capacity keeps 8 * blk
      // within 32 bits): the stores take their base from scalar registers.
      st_stream(a.job[j].codes + (uint32_t)(8u * blk[it]), c);
      a.job[j].scales[(uint32_t)blk[it]] = (uint8_t)S;
    }
    // Keep blocks from being interleaved by the scheduler: hoisting every
    // block's unpacked values at once would exceed the register budget.
    __builtin_amdgcn_sched_barrier(0);
  }
  if (threadIdx.x == 0 && fused_last_to_finish(ctrl, slot))
    for (int j = 0; j < njobs; ++j) *a.job[j].tensor_scale = published_scale(ctrl, s_st[j]);
}

template <bool kBF16, bool kRHT, bool kContig, bool kPre = false>
__global__ __launch_bounds__(kThreads) void row_amax_kernel(RowArgs a) {
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;
  const float clip = (!kBF16 && a.clip) ? *a.clip : 0.0f;
  const int lane = threadIdx.x & 63;
  const uint64_t nseg = (a.nblocks + 63) / 64;
  const uint64_t nwaves = (uint64_t)gridDim.x * (kThreads / 64);
  uint32_t m = 0;
  for (uint64_t s0 = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); s0 < nseg;
       s0 += kBatch * nwaves) {
    RawBlock<kBF16> raw[kBatch];
    uint64_t blk[kBatch];
    load_segments<kBF16, kContig, false>(a, s0, nwaves, lane, raw, blk);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      uint32_t bm;
      if constexpr (kBF16 && !kRHT && !kPre) {
        bm = raw[i].max_abs_bf16();
      } else {
        float v[16];
        raw[i].values(v);
        if constexpr (kPre) (void)sqrt_demean16(v);
        if (!kBF16 && a.clip) {
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = clamp_abs(v[j], clip);
        }
        if (kRHT) {
          rht16_unscaled(v, mask);
          bm = quarter_max_bits(max_abs16(v));
        } else {
          bm = max_abs16(v);
        }
      }
      m = max(m, blk[i] < a.nblocks ? bm : 0u);
    }
  }
  block_amax_commit(m, a.ctrl);
}

template <bool kBF16, bool kRHT, bool kSR, bool kContig, bool kPre = false>
__global__ __launch_bounds__(kThreads) void row_encode_kernel(RowArgs a) {
  __shared__ float recip[128];
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;
  const float amax = __uint_as_float(load_amax(a.ctrl));
  const float st = amax / 2688.0f;
  const float d6 = 6.0f * st;
  const float clip = (!kBF16 && a.clip) ? *a.clip : 0.0f;
  build_recip_table(recip, st);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const uint64_t nseg = (a.nblocks + 63) / 64;
  const uint64_t nwaves = (uint64_t)gridDim.x * (kThreads / 64);
  for (uint64_t s0 = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); s0 < nseg;
       s0 += kBatch * nwaves) {
    RawBlock<kBF16> raw[kBatch];
    uint64_t blk[kBatch];
    load_segments<kBF16, kContig, true>(a, s0, nwaves, lane, raw, blk);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (blk[i] < a.nblocks) {
        float v[16];
        raw[i].values(v);
        if constexpr (kPre) a.means[blk[i]] = (uint16_t)sqrt_demean16(v);
        if (!kBF16 && a.clip) {
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = clamp_abs(v[j], clip);
        }
        if (kRHT) rht16(v, mask);
        row_store_block<kSR>(a, blk[i], v, block_scale_code(max_abs16(v), st, d6), recip);
      }
    }
  }
  encode_finish(a.ctrl, a.tensor_scale, st);
}

// ---------------------------------------------------------------------------
// Transposing kernels
// ---------------------------------------------------------------------------

// Workgroup tile: 256 input rows (16 row blocks) x 128 input columns (16
// groups of 8).  Lane (cg, rb) = (tid % 16, tid / 16) owns 8 columns x 16
// rows = 8 blocks of the transposed view.  For each input row, the 16 lanes
// of one row block read 256 contiguous bytes.  Codes of the whole tile (128
// transposed rows x 128 bytes) are staged in LDS and written out as whole
// lines.
constexpr int kColTileRB = 16;   // row blocks per tile
constexpr int kColTileCG = 16;   // column groups per tile

struct ColArgs {
  const void *x;
  int64_t batch, R, C, ld, bstride;  // input [batch][R][C]; R % 16 == 0
  int64_t tiles_r, tiles_c;          // ceil(R / 256), ceil(C / 128)
  bool vec_ok;                       // rows and batches start on 16-byte boundaries
  uint8_t *codes, *scales;
  float *tensor_scale;
  QuantCtrl *ctrl;
  uint64_t sr_seed, rht_seed;
  uint32_t sr_stream;
  const float *clip;                 // dual encode of FP32 only: clamp to [-*clip, *clip] first
};

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

// Load a lane's 16 rows x 8 columns.  `full` (uniform over the workgroup:
// the whole tile lies inside the tensor's columns and rows start on 16-byte
// boundaries) takes one or two 16-byte loads per row, all issued before any
// is waited for; otherwise element loads with columns at or beyond C read as
// zero.  Lanes outside the tensor pass clamped, in-bounds coordinates and
// ignore what they load.
template <bool kBF16>
__device__ __forceinline__ void col_load(const ColArgs &a, int64_t b, int64_t rb, int64_t cg, bool full,
                                         ColTile<kBF16> &t) {
  const int64_t c0 = 8 * cg;
  const uint8_t *base = static_cast<const uint8_t *>(a.x) + (b * a.bstride + 16 * rb * a.ld + c0) * (kBF16 ? 2 : 4);
  const int64_t ldb = a.ld * (kBF16 ? 2 : 4);
  if (full) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint8_t *p = base + j * ldb;
      const uint4 q = *reinterpret_cast<const uint4 *>(p);
      t.w[j][0] = q.x; t.w[j][1] = q.y; t.w[j][2] = q.z; t.w[j][3] = q.w;
      if (!kBF16) {
        const uint4 q1 = *reinterpret_cast<const uint4 *>(p + 16);
        t.w[j][4] = q1.x; t.w[j][5] = q1.y; t.w[j][6] = q1.z; t.w[j][7] = q1.w;
      }
    }
    return;
  }
  // Element loads at clamped column offsets (c0 < C), masked afterwards.
  const int lim = (int)min((int64_t)7, a.C - 1 - c0);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (kBF16) {
      const uint16_t *p = reinterpret_cast<const uint16_t *>(base + j * ldb);
      uint32_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = p[min(i, lim)];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = i <= lim ? e[i] : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) t.w[j][i] = e[2 * i] | (e[2 * i + 1] << 16);
    } else {
      const uint32_t *p = reinterpret_cast<const uint32_t *>(base + j * ldb);
#pragma unroll
      for (int i = 0; i < 8; ++i) t.w[j][i] = p[min(i, lim)];
#pragma unroll
      for (int i = 0; i < 8; ++i) t.w[j][i] = i <= lim ? t.w[j][i] : 0u;
    }
  }
}

// A lane's unit of the two-pass tiles: row block rb, column group cg; ld_rb
// and ld_cg are the same clamped into the tensor (what the lane loads).
struct ColLane {
  int64_t b, tr, tc, rb, cg, ld_rb, ld_cg;
  bool valid, full;
};

__device__ __forceinline__ ColLane col_lane(const ColArgs &a) {
  ColLane l;
  const int64_t bid = blockIdx.x;
  l.tc = bid % a.tiles_c;
  const int64_t t = bid / a.tiles_c;
  l.tr = t % a.tiles_r;
  l.b = t / a.tiles_r;
  l.cg = l.tc * kColTileCG + (threadIdx.x % kColTileCG);
  l.rb = l.tr * kColTileRB + (threadIdx.x / kColTileCG);
  l.valid = l.rb < a.R / 16 && 8 * l.cg < a.C;
  l.ld_rb = min(l.rb, a.R / 16 - 1);
  l.ld_cg = min(l.cg, (a.C - 1) / 8);
  l.full = a.vec_ok && (l.tc + 1) * (8 * kColTileCG) <= a.C;
  return l;
}

template <bool kBF16, bool kRHT>
__global__ __launch_bounds__(kThreads) void col_amax_kernel(ColArgs a) {
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;
  const ColLane l = col_lane(a);
  uint32_t m = 0;
  ColTile<kBF16> t;
  col_load<kBF16>(a, l.b, l.ld_rb, l.ld_cg, l.full, t);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = t.at(j, e);
    if (kRHT) {
      rht16_unscaled(v, mask);
      m = max(m, quarter_max_bits(max_abs16(v)));  // columns past C hold zeros
    } else {
      m = max(m, max_abs16(v));
    }
  }
  block_amax_commit(l.valid ? m : 0u, a.ctrl);
}

template <bool kBF16, bool kRHT, bool kSR>
__global__ __launch_bounds__(kThreads) void col_encode_kernel(ColArgs a) {
  __shared__ float recip[128];
  // [tile column][row block], rows padded by one entry against bank conflicts
  __shared__ uint2 tile_codes[kColTileCG * 8][kColTileRB + 1];
  __shared__ uint8_t tile_scales[kColTileCG * 8][kColTileRB + 4];
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;
  const float amax = __uint_as_float(load_amax(a.ctrl));
  const float st = amax / 2688.0f;
  const float d6 = 6.0f * st;
  build_recip_table(recip, st);
  __syncthreads();
  const ColLane l = col_lane(a);
  const int cgl = threadIdx.x % kColTileCG, rbl = threadIdx.x / kColTileCG;
  ColTile<kBF16> t;
  col_load<kBF16>(a, l.b, l.ld_rb, l.ld_cg, l.full, t);
  if (l.valid) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t c = 8 * l.cg + e;  // row of the transposed view
      if (c >= a.C) break;
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = t.at(j, e);
      if (kRHT) rht16(v, mask);
      const uint32_t S = block_scale_code(max_abs16(v), st, d6);
      const int64_t vrow = l.b * a.C + c;  // row index in the [batch*C][R] view
      tile_codes[cgl * 8 + e][rbl] = encode16<kSR>(v, recip[S], (uint64_t)(vrow * a.R + 16 * l.rb), a.sr_stream,
                                                   a.sr_seed);
      tile_scales[cgl * 8 + e][rbl] = (uint8_t)S;
    }
  }
  __syncthreads();
  // Write out: 128 transposed rows x 16 row blocks of 8 code bytes and one
  // scale byte; consecutive threads take consecutive row blocks of a row.
  const int64_t RB = a.R / 16;
  const int64_t rb_n = min((int64_t)kColTileRB, RB - l.tr * kColTileRB);
  for (int i = threadIdx.x; i < kColTileCG * 8 * kColTileRB; i += kThreads) {
    const int tcol = i / kColTileRB, trb = i % kColTileRB;
    const int64_t c = l.tc * kColTileCG * 8 + tcol;
    if (c < a.C && trb < rb_n) {
      const int64_t vrow = l.b * a.C + c;
      const int64_t rb = l.tr * kColTileRB + trb;
      st_stream(a.codes + vrow * (a.R / 2) + 8 * rb, tile_codes[tcol][trb]);
      a.scales[vrow * RB + rb] = tile_scales[tcol][trb];
    }
  }
  encode_finish(a.ctrl, a.tensor_scale, st);
}

// Both orientations from one read (encode pass of the dual quantize): the
// tile and lane layout of col_encode_kernel, whose transposed view it writes
// the same way; the same registers then give the view along the columns.  A
// 16-column block of input row r is split over this lane (8 columns) and
// its neighbour (lane ^ 1, the next column group): the block maximum takes
// one lane-pair exchange, each lane encodes its 8 elements with the shared
// block scale and stores them as 4 contiguous code bytes (the 16 lanes of a
// row group write 64 contiguous bytes).  Without the transform both views
// have the same tensor maximum, hence one tensor scale.
struct DualArgs {
  ColArgs c;                     // input, tiles, the transposed view and its stream
  uint8_t *rcodes, *rscales;     // the view along the columns: [batch][R][C/2], [batch][R][C/16]
  float *rtensor_scale;
  uint64_t r_seed;
  uint32_t r_stream;
};

template <bool kBF16, bool kColSR, bool kRowSR>
__global__ __launch_bounds__(kThreads) void dual_encode_kernel(DualArgs d) {
  const ColArgs &a = d.c;
  __shared__ float recip[128];
  __shared__ uint2 tile_codes[kColTileCG * 8][kColTileRB + 1];
  __shared__ uint8_t tile_scales[kColTileCG * 8][kColTileRB + 4];
  const float amax = __uint_as_float(load_amax(a.ctrl));
  const float st = amax / 2688.0f;
  const float d6 = 6.0f * st;
  build_recip_table(recip, st);
  __syncthreads();
  const ColLane l = col_lane(a);
  const int cgl = threadIdx.x % kColTileCG, rbl = threadIdx.x / kColTileCG;
  ColTile<kBF16> t;
  col_load<kBF16>(a, l.b, l.ld_rb, l.ld_cg, l.full, t);
  if constexpr (!kBF16) {
    if (a.clip) {
      const float c = *a.clip;
#pragma unroll
      for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) t.w[j][e] = __float_as_uint(clamp_abs(__uint_as_float(t.w[j][e]), c));
    }
  }
  // The transposed view, staged in LDS.
  if (l.valid) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t c = 8 * l.cg + e;  // row of the transposed view
      if (c >= a.C) break;
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = t.at(j, e);
      const uint32_t S = block_scale_code(max_abs16(v), st, d6);
      const int64_t vrow = l.b * a.C + c;
      tile_codes[cgl * 8 + e][rbl] = encode16<kColSR>(v, recip[S], (uint64_t)(vrow * a.R + 16 * l.rb), a.sr_stream,
                                                      a.sr_seed);
      tile_scales[cgl * 8 + e][rbl] = (uint8_t)S;
    }
  }
  // The view along the columns, stored directly.  Column groups come in
  // pairs that are both inside or both outside the tensor (C % 16 == 0), so
  // the pair exchange below never mixes a valid lane with an invalid one;
  // every lane takes part in it.
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = t.at(j, i);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, abs_bits(v[i]));
    m = max(m, lane_xor1(m));
    const uint32_t S = block_scale_code(m, st, d6);
    const float r = recip[S];
    if (l.valid) {
      const int64_t row = l.b * a.R + 16 * l.rb + j;
      const int64_t n0 = row * a.C + 8 * l.cg;  // logical index of this lane's first element
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = v[i] * r;
      uint32_t w;
      if (kRowSR) {
        const u32x4 rr = sr_block((uint64_t)n0 / 8, d.r_stream, d.r_seed);
        w = e2m1_sr8(q, rr.x, rr.y, rr.z, rr.w);
      } else {
        w = e2m1_rne8(q);
      }
      *reinterpret_cast<uint32_t *>(d.rcodes + row * (a.C / 2) + 4 * l.cg) = w;
      if ((l.cg & 1) == 0) d.rscales[row * (a.C / 16) + l.cg / 2] = (uint8_t)S;
    }
  }
  __syncthreads();
  // Write out the transposed tile: 128 transposed rows x 16 row blocks.
  const int64_t RB = a.R / 16;
  const int64_t rb_n = min((int64_t)kColTileRB, RB - l.tr * kColTileRB);
  for (int i = threadIdx.x; i < kColTileCG * 8 * kColTileRB; i += kThreads) {
    const int tcol = i / kColTileRB, trb = i % kColTileRB;
    const int64_t c = l.tc * kColTileCG * 8 + tcol;
    if (c < a.C && trb < rb_n) {
      const int64_t vrow = l.b * a.C + c;
      const int64_t rb = l.tr * kColTileRB + trb;
      st_stream(a.codes + vrow * (a.R / 2) + 8 * rb, tile_codes[tcol][trb]);
      a.scales[vrow * RB + rb] = tile_scales[tcol][trb];
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *d.rtensor_scale = st;
  encode_finish(a.ctrl, a.tensor_scale, st);
}

// Single-pass transposing quantize (BF16): at most one workgroup per CU, each
// covering 16 kRB input rows x 128 columns, i.e. kRB x 16 units of 16 rows
// x 8 columns, one unit per thread held in registers (64 dwords); kRB = 64
// (1024 threads) for large tensors, 32 (512 threads, twice the workgroups)
// where the grid of 64-row-block tiles would leave CUs idle.  Phase 1
// takes the eight column blocks' maxima (after the transform), then the grid
// barrier of the row kernel yields the tensor max; phase 2 re-derives each
// column block from the held words and encodes it exactly as
// col_encode_kernel does, staging the tile's codes in LDS so each transposed
// row gets 512 contiguous bytes.  The input is read once.
constexpr int kColFusedCG = 16;  // column groups per tile

template <int kRB, bool kRHT, bool kSR>
__global__ __launch_bounds__(kRB * kColFusedCG) void col_fused_kernel(ColArgs a) {
  constexpr int kColFusedRB = kRB;  // row blocks per tile
  constexpr int kColFusedThreads = kRB * kColFusedCG;
  __shared__ float recip[128];
  __shared__ uint2 tile_codes[kColFusedCG * 8][kColFusedRB + 1];
  __shared__ uint8_t tile_scales[kColFusedCG * 8][kColFusedRB + 4];
  __shared__ uint32_t part[kColFusedThreads / 64];
  __shared__ unsigned long long s_epoch;
  __shared__ float s_st;
  QuantCtrl *ctrl = a.ctrl;
  const int slot = blockIdx.x & 7;
  // The epoch cannot advance before this workgroup arrives: race free.
  if (threadIdx.x == 0) s_epoch = atomic_load_dev(&ctrl->release.v);
  const uint32_t mask = kRHT ? rht_sign_mask(a.rht_seed) : 0u;

  const int64_t bid = blockIdx.x;
  const int64_t tc = bid % a.tiles_c, trb = bid / a.tiles_c;
  const int64_t tr = trb % a.tiles_r, b = trb / a.tiles_r;
  const int cgl = threadIdx.x % kColFusedCG, rbl = threadIdx.x / kColFusedCG;
  const int64_t cg = tc * kColFusedCG + cgl, rb = tr * kColFusedRB + rbl;
  const bool valid = rb < a.R / 16 && 8 * cg < a.C;
  const bool full = a.vec_ok && (tc + 1) * (8 * kColFusedCG) <= a.C;

  // Phase 1: load the unit (clamped into the tensor for lanes outside it,
  // whose maxima are then dropped), block maxima of its (transformed)
  // columns.
  ColTile<true> t;
  col_load<true>(a, b, min(rb, a.R / 16 - 1), min(cg, (a.C - 1) / 8), full, t);
  uint32_t bm[8];
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = t.at(j, e);
    if (kRHT) {
      rht16_unscaled(v, mask);
      bm[e] = quarter_max_bits(max_abs16(v));  // columns past C hold zeros: maximum 0
    } else {
      bm[e] = max_abs16(v);
    }
    m = max(m, valid ? bm[e] : 0u);
    // One column's unpacked values at a time: the unit's 64 words and the
    // eight maxima are what the register budget holds across the barrier.
    __builtin_amdgcn_sched_barrier(0);
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long e = s_epoch;
    if (blockIdx.x == 0) {  // slots of the next epoch: unused since the call before this one ended
#pragma unroll
      for (int i = 0; i < 8; ++i) atomic_store_dev(&ctrl->amax[(e + 1) & 1][i].v, 0u);
    }
    uint32_t wm = part[0];
    for (int w = 1; w < kColFusedThreads / 64; ++w) wm = max(wm, part[w]);
    const uint32_t prev =
        __hip_atomic_fetch_max(&ctrl->amax[e & 1][slot].v, wm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_for(prev);  // the max is performed before this workgroup counts as arrived
    (void)fused_arrive_wait(ctrl, e, slot);
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, atomic_load_dev(&ctrl->amax[e & 1][i].v));
    s_st = __uint_as_float(am) / 2688.0f;
  }
  __syncthreads();
  const float st = s_st;
  const float d6 = 6.0f * st;
  build_recip_table(recip, st);
  __syncthreads();

  // Phase 2: encode from registers into the LDS tile.  The words are hidden
  // from value numbering so that phase 1's unpacked values are recomputed
  // here rather than kept alive across the barrier.
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(t.w[j][i]));
  // Element, code and scale indices in 32 bits: the grid covers at most one
  // tile per CU, so the whole tensor has fewer than 2^25 elements.
  const uint32_t R32 = (uint32_t)a.R, C32 = (uint32_t)a.C;
  if (valid) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t c = 8u * (uint32_t)cg + e;  // row of the transposed view
      if (c >= C32) break;
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = t.at(j, e);
      if (kRHT) rht16(v, mask);
      const uint32_t S = block_scale_code(bm[e], st, d6);
      const uint32_t vrow = (uint32_t)b * C32 + c;  // row index in the [batch*C][R] view
      tile_codes[cgl * 8 + e][rbl] =
          encode16<kSR>(v, recip[S], (uint64_t)(vrow * R32 + 16u * (uint32_t)rb), a.sr_stream, a.sr_seed);
      tile_scales[cgl * 8 + e][rbl] = (uint8_t)S;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  // Write out: 128 transposed rows x kRB row blocks of 8 code bytes and one
  // scale byte; consecutive threads take consecutive row blocks of a row.
  const uint32_t RB = R32 / 16;
  const uint32_t rb_n = min((uint32_t)kColFusedRB, RB - (uint32_t)tr * kColFusedRB);
  for (int i = threadIdx.x; i < kColFusedCG * 8 * kColFusedRB; i += kColFusedThreads) {
    const uint32_t tcol = i / kColFusedRB, trbl = i % kColFusedRB;
    const uint32_t c = (uint32_t)tc * kColFusedCG * 8 + tcol;
    if (c < C32 && trbl < rb_n) {
      const uint32_t vrow = (uint32_t)b * C32 + c;
      const uint32_t r = (uint32_t)tr * kColFusedRB + trbl;
      st_stream(a.codes + (vrow * (R32 / 2) + 8u * r), tile_codes[tcol][trbl]);
      a.scales[vrow * RB + r] = tile_scales[tcol][trbl];
    }
  }
  if (threadIdx.x == 0 && fused_last_to_finish(ctrl, slot)) *a.tensor_scale = published_scale(ctrl, st);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

int grid_for(uint64_t items, int threads, uint64_t cap) {
  const uint64_t want = (items + threads - 1) / threads;
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

// Device properties the single-pass launchers need, queried once per device
// and kept (a device's CU count and a kernel's occupancy do not change
// while the process runs).  Concurrent first calls may both query; they
// store the same value.
constexpr int kMaxDevices = 64;

int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

int cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  const int dev = current_device();
  if (dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Resident workgroups per CU of kKernel at kThreadsPerGroup threads (0 if
// the query fails), cached per device; one table per kernel instance.
template <auto kKernel, int kThreadsPerGroup>
int occupancy() {
  static std::atomic<int> cache[kMaxDevices];  // value + 1, 0 = unknown
  const int dev = current_device();
  if (dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v - 1;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kKernel, kThreadsPerGroup, 0) != hipSuccess) return 0;
  if (dev < kMaxDevices) cache[dev].store(per_cu + 1, std::memory_order_relaxed);
  return per_cu;
}

// Single-pass row-wise quantize of the jobs in `a` if they fit the on-chip
// capacity of a co-resident grid; returns false (nothing launched) otherwise.
template <bool kBF16, bool kRHT, bool kSR>
bool try_row_fused(FusedArgs a, hipStream_t s, hipError_t &err) {
  const int cus = cu_count();
  if (cus <= 0) return false;
  auto kernel = row_fused_kernel<kBF16, kRHT, kSR>;
  if (occupancy<row_fused_kernel<kBF16, kRHT, kSR>, kFusedThreads>() < 1) return false;
  const uint64_t grid = (uint64_t)cus;
  const uint64_t nwaves = grid * (kFusedThreads / 64);
  const uint64_t iters = (a.nseg + nwaves - 1) / nwaves;
  if (iters > (uint64_t)Fused<kBF16, kRHT, kSR>::kMaxBlocks) return false;
  a.nseg_iters = (uint32_t)iters;
  // A plain launch: with one workgroup per CU every workgroup becomes
  // resident once kernels already running on other streams drain, so the
  // grid barrier completes; the bounded wait only guards against a kernel
  // that holds CUs indefinitely.  (The cooperative-launch API gives the same
  // guarantee up front but costs ~18 us per call on MI355X.)
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kFusedThreads), 0, s, a);
  err = hipGetLastError();
  return err == hipSuccess;
}

// The single-pass arguments of one contiguous tensor.
FusedArgs fused_single(const RowArgs &r) {
  FusedArgs a{};
  a.job[0].x = r.x;
  a.job[0].nblocks = r.nblocks;
  a.job[0].seg_begin = 0;
  a.job[0].codes = r.codes;
  a.job[0].scales = r.scales;
  a.job[0].tensor_scale = r.tensor_scale;
  a.job[0].amax = r.ctrl->amax;
  a.njobs = 1;
  a.nseg = (r.nblocks + 63) / 64;
  a.ctrl = r.ctrl;
  a.sr_seed = r.sr_seed;
  a.rht_seed = r.rht_seed;
  a.sr_stream = r.sr_stream;
  return a;
}

template <bool kBF16, bool kRHT, bool kSR, bool kContig>
hipError_t run_row_two_pass(const RowArgs &a, hipStream_t s) {
  const int g = grid_for((a.nblocks + 63) / 64, (kThreads / 64) * kBatch, 256ull * 4);
  hipLaunchKernelGGL((row_amax_kernel<kBF16, kRHT, kContig>), dim3(g), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((row_encode_kernel<kBF16, kRHT, kSR, kContig>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool kBF16, bool kRHT, bool kSR>
hipError_t run_row(const RowArgs &a, bool contig, hipStream_t s) {
  if (contig && !a.clip) {
    hipError_t err = hipSuccess;
    if (try_row_fused<kBF16, kRHT, kSR>(fused_single(a), s, err)) return hipSuccess;
    if (err != hipSuccess) return err;  // a launch that was refused is reported, not retried
    return run_row_two_pass<kBF16, kRHT, kSR, true>(a, s);
  }
  return run_row_two_pass<kBF16, kRHT, kSR, false>(a, s);
}

template <bool kBF16>
hipError_t dispatch_row(const RowArgs &a, bool rht, bool sr, bool contig, hipStream_t s) {
  if (rht) return sr ? run_row<kBF16, true, true>(a, contig, s) : run_row<kBF16, true, false>(a, contig, s);
  return sr ? run_row<kBF16, false, true>(a, contig, s) : run_row<kBF16, false, false>(a, contig, s);
}

// Single-pass transposing quantize if a grid of 16 kRB-row x 128-column
// tiles fits one workgroup per CU (BF16 only: an FP32 unit would not fit the
// register budget): 512-row tiles when those fit (more workgroups for the
// same tensor), else 1024-row tiles.  Returns false (nothing launched) if
// neither fits.
template <int kRB, bool kRHT, bool kSR>
bool launch_col_fused(ColArgs a, int cus, hipStream_t s, hipError_t &err) {
  constexpr int kThreadsPerGroup = kRB * kColFusedCG;
  if (occupancy<col_fused_kernel<kRB, kRHT, kSR>, kThreadsPerGroup>() < 1) return false;
  a.tiles_r = (a.R / 16 + kRB - 1) / kRB;
  a.tiles_c = (a.C + 8 * kColFusedCG - 1) / (8 * kColFusedCG);
  const int64_t grid = a.batch * a.tiles_r * a.tiles_c;
  if (grid < 1 || grid > (int64_t)cus) return false;
  // A plain launch: with at most one workgroup per CU every workgroup
  // becomes resident, so the grid barrier completes (bounded wait besides).
  hipLaunchKernelGGL((col_fused_kernel<kRB, kRHT, kSR>), dim3((unsigned)grid), dim3(kThreadsPerGroup), 0, s, a);
  err = hipGetLastError();
  return err == hipSuccess;
}

template <bool kRHT, bool kSR>
bool try_col_fused(const ColArgs &a, hipStream_t s, hipError_t &err) {
  const int cus = cu_count();
  if (cus <= 0) return false;
  if (launch_col_fused<32, kRHT, kSR>(a, cus, s, err)) return true;
  return err == hipSuccess && launch_col_fused<64, kRHT, kSR>(a, cus, s, err);
}

template <bool kBF16, bool kRHT, bool kSR>
hipError_t run_col(const ColArgs &a, hipStream_t s) {
  if constexpr (kBF16) {
    hipError_t err = hipSuccess;
    if (try_col_fused<kRHT, kSR>(a, s, err)) return hipSuccess;
    if (err != hipSuccess) return err;
  }
  const uint64_t g = (uint64_t)(a.batch * a.tiles_r * a.tiles_c);
  if (g > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL((col_amax_kernel<kBF16, kRHT>), dim3((unsigned)g), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((col_encode_kernel<kBF16, kRHT, kSR>), dim3((unsigned)g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool kBF16>
hipError_t dispatch_col(const ColArgs &a, bool rht, bool sr, hipStream_t s) {
  if (rht) return sr ? run_col<kBF16, true, true>(a, s) : run_col<kBF16, true, false>(a, s);
  return sr ? run_col<kBF16, false, true>(a, s) : run_col<kBF16, false, false>(a, s);
}

__global__ void store_zero_scale(float *p) { *p = 0.0f; }

template <bool kBF16>
bool dispatch_group_fused(const FusedArgs &a, bool rht, bool sr, hipStream_t s, hipError_t &err) {
  if (rht) return sr ? try_row_fused<kBF16, true, true>(a, s, err) : try_row_fused<kBF16, true, false>(a, s, err);
  return sr ? try_row_fused<kBF16, false, true>(a, s, err) : try_row_fused<kBF16, false, false>(a, s, err);
}

}  // namespace

nvfp4_status launch_quantize_group(const QuantGroupProblem &p, hipStream_t s) {
  // One launch when every tensor is contiguous and all fit the single-pass
  // capacity together; otherwise the tensors one after the other.
  FusedArgs a{};
  bool contig = true;
  uint64_t seg = 0;
  int n = 0;
  for (int i = 0; i < p.njobs; ++i) {
    const QuantProblem &q = p.job[i];
    if (q.batch == 0 || q.rows == 0 || q.cols == 0) continue;
    contig = contig && q.ld == q.cols && (q.batch == 1 || q.bstride == q.rows * q.cols);
    RowJob &j = a.job[n];
    j.x = q.x;
    j.nblocks = (uint64_t)(q.batch * q.rows * q.cols / 16);
    j.seg_begin = seg;
    j.codes = q.codes;
    j.scales = q.scales;
    j.tensor_scale = q.tensor_scale;
    seg += (j.nblocks + 63) / 64;
    ++n;
  }
  for (int i = 0; i < kMaxGroup; ++i) a.job[i].amax = p.amax[i];  // all four, see row_fused_kernel
  if (contig && n > 0) {
    a.njobs = n;
    a.nseg = seg;
    a.ctrl = p.ctrl_group;
    a.sr_seed = p.job[0].sr_seed;
    a.rht_seed = p.job[0].rht_seed;
    a.sr_stream = p.job[0].sr_stream;
    hipError_t err = hipSuccess;
    const bool launched = p.job[0].bf16 ? dispatch_group_fused<true>(a, p.job[0].rht, p.job[0].sr, s, err)
                                        : dispatch_group_fused<false>(a, p.job[0].rht, p.job[0].sr, s, err);
    if (launched) {
      for (int i = 0; i < p.njobs; ++i) {  // empty tensors: tensor scale 0
        const QuantProblem &q = p.job[i];
        if (q.batch == 0 || q.rows == 0 || q.cols == 0)
          hipLaunchKernelGGL(store_zero_scale, dim3(1), dim3(1), 0, s, q.tensor_scale);
      }
      return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
    }
    if (err != hipSuccess) return NVFP4_EHIP;
  }
  for (int i = 0; i < p.njobs; ++i) {
    QuantProblem q = p.job[i];
    q.ctrl = p.ctrl_seq;
    const nvfp4_status st = launch_quantize(q, s);
    if (st != NVFP4_OK) return st;
  }
  return NVFP4_OK;
}

namespace {

// Reconstruction of a quantized optimizer state, one 16-element block per
// lane (blocks in row-major order over [rows][cols / 16]): x_j =
// fl(E2M1 * E4M3 * s_t) (the first product is exact), the inverse transform
// (1/4) D H (butterflies with span 1, 2, 4, 8, then the exact product by 1/4,
// then the signs), and for the second moment s_j = fl(x_j + mu), v_j =
// fl(s_j * s_j).  Output rows have stride ld (floats).
struct StateDecodeArgs {
  const uint8_t *codes, *scales;
  const float *tensor_scale;
  const uint16_t *means;  // second moment only
  float *out;
  uint64_t nblocks, bpr;
  int64_t ld;
  uint64_t rht_seed;
};

// One thread per 16-element block, 256 consecutive blocks per workgroup
// and round.  A thread's block is 64 contiguous output bytes, so storing it
// directly would have every store instruction touch 64 partial lines; the
// round's blocks are staged in LDS instead and written back as consecutive
// 16-byte pieces by consecutive threads.
constexpr int kDecodeBlocks = 256;

template <bool kSecond>
__global__ __launch_bounds__(kDecodeBlocks) void state_decode_kernel(StateDecodeArgs a) {
  __shared__ float4 stage[kDecodeBlocks * 4];
  const uint32_t mask = rht_sign_mask(a.rht_seed);
  const float st = *a.tensor_scale;
  for (uint64_t base = (uint64_t)blockIdx.x * kDecodeBlocks; base < a.nblocks;
       base += (uint64_t)gridDim.x * kDecodeBlocks) {
    const uint64_t blk = base + threadIdx.x;
    if (blk < a.nblocks) {
      const uint2 c = *reinterpret_cast<const uint2 *>(a.codes + 8 * blk);
      const float sc = e4m3_value(a.scales[blk]);
      // E2M1 values of the block (scale 1), then H on them: every partial
      // sum is a multiple of 1/2 no larger than 96 in magnitude, so exact.
      float v[16];
      const float2_v p[8] = {
          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 0), __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 1),
          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 2), __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 3),
          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 0), __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 1),
          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 2), __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 3)};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[2 * k] = p[k][0];
        v[2 * k + 1] = p[k][1];
      }
#pragma unroll
      for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (i & h) continue;
          const float x = v[i], y = v[i + h];
          v[i] = x + y;
          v[i + h] = x - y;
        }
      }
      // (1/4) E4M3 is exact, and so is its product with a sum above (at
      // most 12 significant bits); the tensor scale rounds once; then the
      // signs.  A zero sum is taken as +0 (the sums of -0 codes would give
      // -0), so a zero result carries the sign of the diagonal alone.
      const float q4 = sc * 0.25f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float z = v[j] + 0.0f;
        v[j] = __uint_as_float(__float_as_uint((z * q4) * st) ^ (((mask >> j) & 1u) << 31));
      }
      if constexpr (kSecond) {
        const float mu = __uint_as_float((uint32_t)a.means[blk] << 16);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float sj = v[j] + mu;
          v[j] = sj * sj;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        stage[4 * threadIdx.x + q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = threadIdx.x + kDecodeBlocks * i;  // 16-byte piece of the round
      const uint64_t b = base + slot / 4;
      if (b < a.nblocks) {
        const uint64_t row = b / a.bpr, cb = b - row * a.bpr;
        *reinterpret_cast<float4 *>(a.out + row * a.ld + 16 * cb + 4 * (slot & 3)) = stage[slot];
      }
    }
    __syncthreads();
  }
}

}  // namespace

nvfp4_status launch_state_encode_second(const QuantProblem &p, uint16_t *means, hipStream_t s) {
  if (p.rows == 0 || p.cols == 0) {
    hipLaunchKernelGGL(store_zero_scale, dim3(1), dim3(1), 0, s, p.tensor_scale);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
  }
  RowArgs a{};
  a.x = p.x;
  a.nblocks = (uint64_t)(p.rows * p.cols / 16);
  a.bpr = (uint64_t)(p.cols / 16);
  a.rows = p.rows;
  a.ld = p.ld;
  a.bstride = p.rows * p.ld;
  a.codes = p.codes;
  a.scales = p.scales;
  a.tensor_scale = p.tensor_scale;
  a.ctrl = p.ctrl;
  a.rht_seed = p.rht_seed;
  a.means = means;
  const int g = grid_for((a.nblocks + 63) / 64, (kThreads / 64) * kBatch, 256ull * 4);
  if (p.ld == p.cols) {
    hipLaunchKernelGGL((row_amax_kernel<false, true, true, true>), dim3(g), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL((row_encode_kernel<false, true, false, true, true>), dim3(g), dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((row_amax_kernel<false, true, false, true>), dim3(g), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL((row_encode_kernel<false, true, false, false, true>), dim3(g), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status launch_state_decode(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                                 const uint16_t *means, float *out, int64_t rows, int64_t cols, int64_t ld,
                                 uint64_t rht_seed, hipStream_t s) {
  if (rows == 0 || cols == 0) return NVFP4_OK;
  StateDecodeArgs a{codes, scales, tensor_scale, means, out, (uint64_t)(rows * cols / 16), (uint64_t)(cols / 16), ld,
                    rht_seed};
  const int g = grid_for(a.nblocks, kDecodeBlocks, 256ull * 16);
  if (means) hipLaunchKernelGGL((state_decode_kernel<true>), dim3(g), dim3(kDecodeBlocks), 0, s, a);
  else hipLaunchKernelGGL((state_decode_kernel<false>), dim3(g), dim3(kDecodeBlocks), 0, s, a);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

namespace {

template <bool kBF16, bool kColSR, bool kRowSR>
hipError_t run_dual(const RowArgs &ra, const DualArgs &d, bool contig, hipStream_t s) {
  // amax over the input (orientation-free), then one encode pass for both views
  const int g = grid_for((ra.nblocks + 63) / 64, (kThreads / 64) * kBatch, 256ull * 4);
  if (contig) hipLaunchKernelGGL((row_amax_kernel<kBF16, false, true>), dim3(g), dim3(kThreads), 0, s, ra);
  else hipLaunchKernelGGL((row_amax_kernel<kBF16, false, false>), dim3(g), dim3(kThreads), 0, s, ra);
  const uint64_t tiles = (uint64_t)(d.c.batch * d.c.tiles_r * d.c.tiles_c);
  if (tiles > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dual_encode_kernel<kBF16, kColSR, kRowSR>), dim3((unsigned)tiles), dim3(kThreads), 0, s, d);
  return hipGetLastError();
}

template <bool kBF16>
hipError_t dispatch_dual(const RowArgs &ra, const DualArgs &d, bool col_sr, bool row_sr, bool contig, hipStream_t s) {
  if (col_sr) return row_sr ? run_dual<kBF16, true, true>(ra, d, contig, s) : run_dual<kBF16, true, false>(ra, d, contig, s);
  return row_sr ? run_dual<kBF16, false, true>(ra, d, contig, s) : run_dual<kBF16, false, false>(ra, d, contig, s);
}

}  // namespace

nvfp4_status launch_quantize_dual(const QuantProblem &row, const QuantProblem &col, hipStream_t s) {
  if (row.batch == 0 || row.rows == 0 || row.cols == 0) {
    hipLaunchKernelGGL(store_zero_scale, dim3(1), dim3(1), 0, s, row.tensor_scale);
    hipLaunchKernelGGL(store_zero_scale, dim3(1), dim3(1), 0, s, col.tensor_scale);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
  }
  if (row.clip && row.bf16) return NVFP4_EUNSUPPORTED;
  RowArgs ra{};
  ra.x = row.x;
  ra.clip = row.clip;
  ra.nblocks = (uint64_t)(row.batch * row.rows * row.cols / 16);
  ra.bpr = (uint64_t)(row.cols / 16);
  ra.rows = row.rows;
  ra.ld = row.ld;
  ra.bstride = row.bstride;
  ra.ctrl = row.ctrl;
  const bool contig = (row.ld == row.cols) && (row.batch == 1 || row.bstride == row.rows * row.ld);
  DualArgs d{};
  ColArgs &a = d.c;
  a.x = row.x;
  a.batch = row.batch;
  a.R = row.rows;
  a.C = row.cols;
  a.ld = row.ld;
  a.bstride = row.bstride;
  a.tiles_r = (row.rows / 16 + kColTileRB - 1) / kColTileRB;
  a.tiles_c = (row.cols + 8 * kColTileCG - 1) / (8 * kColTileCG);
  const int64_t esize = row.bf16 ? 2 : 4;
  a.vec_ok = reinterpret_cast<uintptr_t>(row.x) % 16 == 0 && (row.ld * esize) % 16 == 0 &&
             (row.batch == 1 || (row.bstride * esize) % 16 == 0);
  a.codes = col.codes;
  a.scales = col.scales;
  a.tensor_scale = col.tensor_scale;
  a.ctrl = row.ctrl;
  a.sr_seed = col.sr_seed;
  a.sr_stream = col.sr_stream;
  a.clip = row.clip;
  d.rcodes = row.codes;
  d.rscales = row.scales;
  d.rtensor_scale = row.tensor_scale;
  d.r_seed = row.sr_seed;
  d.r_stream = row.sr_stream;
  const hipError_t err = row.bf16 ? dispatch_dual<true>(ra, d, col.sr, row.sr, contig, s)
                                  : dispatch_dual<false>(ra, d, col.sr, row.sr, contig, s);
  return err == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status launch_quantize(const QuantProblem &p, hipStream_t s) {
  const int64_t qr = p.along_rows ? p.cols : p.rows;
  const int64_t qc = p.along_rows ? p.rows : p.cols;
  if (p.batch == 0 || qr == 0 || qc == 0) {
    hipLaunchKernelGGL(store_zero_scale, dim3(1), dim3(1), 0, s, p.tensor_scale);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
  }
  if (p.clip && (p.bf16 || p.along_rows)) return NVFP4_EUNSUPPORTED;
  hipError_t err;
  if (!p.along_rows) {
    RowArgs a{};
    a.clip = p.clip;
    a.x = p.x;
    a.nblocks = (uint64_t)(p.batch * p.rows * p.cols / 16);
    a.bpr = (uint64_t)(p.cols / 16);
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
    err = p.bf16 ? dispatch_row<true>(a, p.rht, p.sr, contig, s) : dispatch_row<false>(a, p.rht, p.sr, contig, s);
  } else {
    ColArgs a{};
    a.x = p.x;
    a.batch = p.batch;
    a.R = p.rows;
    a.C = p.cols;
    a.ld = p.ld;
    a.bstride = p.bstride;
    a.tiles_r = (p.rows / 16 + kColTileRB - 1) / kColTileRB;
    a.tiles_c = (p.cols + 8 * kColTileCG - 1) / (8 * kColTileCG);
    const int64_t esize = p.bf16 ? 2 : 4;
    a.vec_ok = reinterpret_cast<uintptr_t>(p.x) % 16 == 0 && (p.ld * esize) % 16 == 0 &&
               (p.batch == 1 || (p.bstride * esize) % 16 == 0);
    a.codes = p.codes;
    a.scales = p.scales;
    a.tensor_scale = p.tensor_scale;
    a.ctrl = p.ctrl;
    a.sr_seed = p.sr_seed;
    a.rht_seed = p.rht_seed;
    a.sr_stream = p.sr_stream;
    err = p.bf16 ? dispatch_col<true>(a, p.rht, p.sr, s) : dispatch_col<false>(a, p.rht, p.sr, s);
  }
  return err == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace nvfp4
