// gemm.hip -- block-scaled NVFP4 GEMM for gfx950.
//
// C[b][i][j] = alpha * sA * sB * sum_k A^[b][i][k] * B^[b][j][k], both operands
// stored as E2M1 codes along K with one E4M3 scale per 16 K-elements: the
// NVFP4 GEMM of weights and activations with wide accumulators that "NVIDIA
// acelera o pre-treinamento de LLM ..." ("Como o Treinamento Mixed-Precision
// Funciona com NVFP4") and "Full-Stack FP4 ..." (section 1) describe.
//
// Exactness: every E2M1 x E4M3 product has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in FP16 (11 bits, normal range down
// to 2^-14).  The kernel decodes codes and scales to FP16 in registers and
// runs v_mfma_f32_32x32x16_f16 with FP32 accumulation; only the FP32
// accumulation order differs from exact arithmetic.  FP16 rather than BF16
// (same MFMA rate on gfx950): the hardware FP4 -> FP16 converter plus one
// packed FP16 multiply by the block scale decode two elements per
// instruction each.  (The converter's own scale operand only honours the
// exponent of its FP32 argument, so it runs at unit scale.)
//
// Tiling: a 256 x (64 * kFragN) output tile per workgroup of 4 wavefronts in
// a 2 x 2 grid, each wavefront owning 128 x (32 * kFragN) = 4 x kFragN MFMA
// tiles, one wavefront per SIMD.  K advances 128 elements (8 scale blocks)
// per step through two LDS stages (64 code bytes + 8 scale bytes per row per
// step).  Within a step, lane half h of a fragment covers K offsets
// [64h, 64h + 64): MFMA sub-step s takes offsets 64h + 8s .. 64h + 8s + 7,
// i.e. one scale block (4h + s/2) per lane.  A and B use the same
// assignment, so each K index meets its partner once.
//
// The decode is the VALU cost (a convert and a packed multiply per two
// elements), and with one wavefront per SIMD it only overlaps the matrix
// pipe when it sits between MFMAs of other operands.  Three main loops:
//  * K % 128 == 0, tiles 256 x 192 / 256 x 128: software pipelined.  The next
//    sub-step is decoded while the current one's MFMAs run (grouped one MFMA
//    to a few VALU instructions), codes are read from LDS half a step ahead,
//    and global_load_lds fills the stage of the step after next, so global
//    latency has a whole step and LDS latency half a step to hide.
//  * K % 128 == 0, tiles 256 x 256: the accumulators fill the AGPR file,
//    which leaves room for double-buffered decoded operands but for one code
//    and one scale buffer only: the same overlap of decode and MFMAs, with
//    each half step's codes read once the previous half's are dead.
//  * Other K: register-staged loads with the K tail read as zero codes and
//    scales (zero products).
// A second kernel runs two wavefronts per SIMD (8 per workgroup, 512 x 192
// or 256 x 384 tiles, three LDS stages); see its section below.  The
// launcher costs every kernel and tile shape by its rounds of workgroups over
// the 256 CUs and picks the cheapest.
//
// Workgroups are mapped to tiles so that each XCD (blockIdx mod 8 under the
// round-robin dispatch) works on a contiguous range of tiles, in groups of
// tile rows (8 for square tiles, 4 where the A tile is the larger), to keep
// A and B panels in that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "device_codec.hpp"
#include "internal.hpp"


namespace nvfp4 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kRowBytes = BK / 2;  // 64 code bytes per row per K step
constexpr int kFragM = 4;          // 32-row A fragments per wavefront
constexpr int kGroupM = 8;         // tile rows per L2 group (square tiles)
// VALU instructions the scheduler places after each MFMA of a pipelined
// sub-step (the decode of the next sub-step); 4 and 5 measured best.
constexpr int kInterleave = 5;
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// LDS placement of the 16-byte code chunk `part` (0..3) of tile row `row`.
// Fragment reads take the same part from 32 consecutive rows; XOR-ing the
// part with row bits spreads those reads over all LDS banks.
__device__ __forceinline__ int chunk_slot(int row, int part) { return row * 4 + (part ^ ((row >> 2) & 3)); }

struct GemmArgs {
  const uint8_t *a_codes, *a_scales;
  const float *a_st;
  const uint8_t *b_codes, *b_scales;
  const float *b_st;
  int64_t M, N, K;
  int tiles_m, tiles_n;
  void *c;
  int64_t ldc, bstride_c;
  float alpha;
  const float *cin;  // optional FP32 addend [batch][M][N] (row stride ldcin), times beta
  int64_t ldcin, bstride_cin;
  float beta;
  // optional low-rank term lr_beta * T L2^T in BF16 (batch 1): T [M][lr_r],
  // L2 [N][lr_r], row-major, lr_r a multiple of 16
  const uint16_t *lr_t, *lr_l2;
  int64_t lr_r;
  float lr_beta;
  // symmetric split-K (A^ A^^T): tiles per side, splits, K steps per split,
  // and the partial tiles [pair * splits + split][BM][BM]
  int sym_t, sym_splits, sym_steps;
  float *sym_part;
  bool ct;      // C stored transposed: tile element (r, c) at c * ldc + r (FP32)
  bool staged;  // FP32 output with an addend or transposed, C and cin 16-byte aligned
                // with strides multiples of 4: full tiles go through the LDS patch
};

// LDS stage: codes [rows][64 B] and scales [rows][8 B] per operand.
template <int kBN>
struct alignas(16) Stage {
  uint8_t a[BM * kRowBytes];
  uint8_t b[kBN * kRowBytes];
  uint2 as[BM];
  uint2 bs[kBN];
};

// global_load_lds of 16 / 4 bytes per lane into the 64 consecutive lane
// slots at LDS byte address `lds` (wavefront-uniform, through M0), from the
// scalar base `base` plus the lane's 32-bit offset.  Written as assembly so
// that the compiler does not track these loads: its own waits for loads that
// write LDS drain all of them before unrelated LDS reads.  Every kernel that
// uses it waits for these loads explicitly (s_waitcnt vmcnt) before the
// barrier that publishes a stage, and issues them only after its last read
// of the stage they refill.  M0 is set in the same statement; nothing else
// in these kernels keeps a value in M0 (checked in the generated code).
template <int kBytes>
__device__ __forceinline__ void dma(const uint8_t *base, uint32_t off, uint32_t lds) {
  if constexpr (kBytes == 16)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory");
}

// Direct global -> LDS loads of one operand's K step (K % 128 == 0): each
// wavefront's global_load_lds fills 64 consecutive lane slots, which keeps
// the row-major [rows][64 B] code and [rows][8 B] scale layout.  Rows past
// the end are clamped; their products only reach output rows never stored.
template <int kRows, bool kOff32>
__device__ __forceinline__ void lds_load_operand(const uint8_t *codes_g, const uint8_t *scales_g,
                                                 int64_t rows, int64_t K, int64_t r0, int64_t k0,
                                                 uint8_t *lds_codes, uint2 *lds_scales, int tid = -1) {
  if (tid < 0) tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t kblocks = K / 16;
  constexpr int kCodeLoads = kRows * 4 / kThreads;  // 16-byte chunks per lane
  constexpr int kScaleLoads = (kRows * 2 + kThreads - 1) / kThreads;  // dwords per lane
  if constexpr (kOff32) {
    // Operands under 2 GiB with fewer than 2^24 rows and code bytes per row:
    // 32-bit offsets and 24-bit products.  A code load's lane takes row
    // 16 (job) + lane / 4, whose swizzle bits (2..3) come from the lane
    // alone; a scale load's lane takes row 32 (job) + lane / 2.
    const int last = (int)(rows - 1 - r0);
    const uint32_t base = (uint32_t)r0, kb2 = (uint32_t)(K / 2), kb16 = (uint32_t)kblocks;
    const uint32_t part16 = 16u * (uint32_t)(chunk_slot(lane >> 2, lane & 3) & 3);
    const uint32_t lds_codes_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_codes);
    const uint32_t lds_scales_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_scales);
#pragma unroll
    for (int i = 0; i < kCodeLoads; ++i) {
      const int job = kCodeLoads * wave + i;
      const uint32_t gr = base + (uint32_t)min(16 * job + (lane >> 2), last);
      dma<16>(codes_g + k0 / 2, __umul24(gr, kb2) + part16, lds_codes_base + 1024u * job);
    }
#pragma unroll
    for (int i = 0; i < kScaleLoads; ++i) {
      const int job = kScaleLoads * wave + i;
      if (64 * job < kRows * 2) {  // wave-uniform
        const uint32_t gr = base + (uint32_t)min(32 * job + (lane >> 1), last);
        if (64 * job + lane < kRows * 2)
          dma<4>(scales_g + k0 / 16, __umul24(gr, kb16) + 4u * (uint32_t)(lane & 1), lds_scales_base + 256u * job);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kCodeLoads; ++i) {
      const int slot = (kCodeLoads * wave + i) * 64;
      const int p = slot + lane;  // physical chunk: row p/4, position p%4
      const int row = p >> 2;
      const int part = (chunk_slot(row, p & 3)) & 3;  // the XOR swizzle is its own inverse
      const int64_t gr = min(r0 + row, rows - 1);
      const uint8_t *src = codes_g + gr * (K / 2) + k0 / 2 + 16 * part;
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(lds_codes + 16 * slot), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kScaleLoads; ++i) {
      const int slot = (kScaleLoads * wave + i) * 64;
      const int p = slot + lane;
      if (slot < kRows * 2) {  // wave-uniform
        const int64_t gr = min(r0 + (p >> 1), rows - 1);
        const uint8_t *src = scales_g + gr * kblocks + k0 / 16 + 4 * (p & 1);
        if (p < kRows * 2)
          __builtin_amdgcn_global_load_lds(src, (lds_void *)(reinterpret_cast<uint8_t *>(lds_scales) + 4 * slot), 4,
                                           0, 0);
      }
    }
  }
}

// Register-staged loads for K % 128 != 0: K blocks past the end read as zero
// codes with zero scales, which contribute exactly 0.
template <int kRows>
struct StagedLoad {
  static constexpr int kChunks = kRows * 4 / kThreads;  // 16-byte code chunks per thread
  uint4 codes[kChunks];
  uint2 scales;
  __device__ __forceinline__ void load(const uint8_t *codes_g, const uint8_t *scales_g, int64_t rows,
                                       int64_t K, int64_t r0, int64_t k0) {
    const int tid = threadIdx.x;
    const int64_t kblocks = K / 16;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int idx = tid + kThreads * i;
      const int64_t gr = min(r0 + (idx >> 2), rows - 1);
      const uint8_t *p = codes_g + gr * (K / 2) + k0 / 2 + 16 * (idx & 3);
      const int64_t kb = k0 / 16 + 2 * (idx & 3);  // blocks kb, kb+1: 8 bytes each
      const uint2 lo = kb < kblocks ? *reinterpret_cast<const uint2 *>(p) : make_uint2(0u, 0u);
      const uint2 hi = kb + 1 < kblocks ? *reinterpret_cast<const uint2 *>(p + 8) : make_uint2(0u, 0u);
      codes[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    uint32_t w[2] = {0u, 0u};
    if (tid < kRows) {
      const int64_t gr = min(r0 + tid, rows - 1);
      const uint8_t *s = scales_g + gr * kblocks + k0 / 16;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (k0 / 16 + i < kblocks) w[i >> 2] |= (uint32_t)s[i] << (8 * (i & 3));
    }
    scales = make_uint2(w[0], w[1]);
  }
  __device__ __forceinline__ void store(uint8_t *lds_codes, uint2 *lds_scales) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int idx = tid + kThreads * i;
      *reinterpret_cast<uint4 *>(lds_codes + chunk_slot(idx >> 2, idx & 3) * 16) = codes[i];
    }
    if (tid < kRows) lds_scales[tid] = scales;
  }
};

// One lane's codes for half a K step: 16 bytes (32 elements, sub-steps
// 4*half .. 4*half + 3) of every fragment it feeds.
template <int kFragN>
struct HalfCodes {
  uint4 a[kFragM], b[kFragN];
};

// One lane's block scales for a K step as FP16 pairs: [f][0] holds blocks
// 4h and 4h + 1 of the step, [f][1] blocks 4h + 2 and 4h + 3.
template <int kFragN>
struct StepScales {
  half2_t a[kFragM][2], b[kFragN][2];
};

struct LaneCoord {
  int wm, wn, h, r32;
};

__device__ __forceinline__ uint32_t word_of(const uint4 &q, int i) {
  return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

template <int kFragN, int kBN>
__device__ __forceinline__ void read_codes(const Stage<kBN> &st, int half, const LaneCoord &c,
                                           HalfCodes<kFragN> &r) {
#pragma unroll
  for (int f = 0; f < kFragM; ++f) {
    const int row = c.wm * 128 + f * 32 + c.r32;
    r.a[f] = *reinterpret_cast<const uint4 *>(st.a + 16 * chunk_slot(row, 2 * c.h + half));
  }
#pragma unroll
  for (int f = 0; f < kFragN; ++f) {
    const int row = c.wn * (32 * kFragN) + f * 32 + c.r32;
    r.b[f] = *reinterpret_cast<const uint4 *>(st.b + 16 * chunk_slot(row, 2 * c.h + half));
  }
}

template <int kFragN, int kBN>
__device__ __forceinline__ void read_scales(const Stage<kBN> &st, const LaneCoord &c, StepScales<kFragN> &sc) {
#pragma unroll
  for (int f = 0; f < kFragM; ++f) {
    const int row = c.wm * 128 + f * 32 + c.r32;
    const uint32_t w = c.h ? st.as[row].y : st.as[row].x;
    sc.a[f][0] = scale_pair_lo(w);
    sc.a[f][1] = scale_pair_lo(w >> 16);
  }
#pragma unroll
  for (int f = 0; f < kFragN; ++f) {
    const int row = c.wn * (32 * kFragN) + f * 32 + c.r32;
    const uint32_t w = c.h ? st.bs[row].y : st.bs[row].x;
    sc.b[f][0] = scale_pair_lo(w);
    sc.b[f][1] = scale_pair_lo(w >> 16);
  }
}

template <int kWord>
__device__ __forceinline__ uint32_t word_at(const uint4 &q) {
  return kWord == 0 ? q.x : kWord == 1 ? q.y : kWord == 2 ? q.z : q.w;
}

// Operands of MFMA sub-step kS (0..7) from the half of the codes holding it.
template <int kS, int kFragN>
__device__ __forceinline__ void decode_substep(const HalfCodes<kFragN> &r, const StepScales<kFragN> &sc,
                                               half8_t (&av)[kFragM], half8_t (&bv)[kFragN]) {
#pragma unroll
  for (int f = 0; f < kFragM; ++f) av[f] = decode8_s256(word_at<kS & 3>(r.a[f]), sc.a[f][kS >> 2][(kS >> 1) & 1]);
#pragma unroll
  for (int f = 0; f < kFragN; ++f) bv[f] = decode8_s256(word_at<kS & 3>(r.b[f]), sc.b[f][kS >> 2][(kS >> 1) & 1]);
}

template <int kFragN>
__device__ __forceinline__ void mfma_substep(floatx16 (&acc)[kFragM][kFragN], const half8_t (&av)[kFragM],
                                             const half8_t (&bv)[kFragN]) {
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
}

// The MFMAs of one sub-step on av/bv, while sub-step kNext is decoded from
// (r, sc) into av/bv's successors.
template <int kNext, int kFragN>
__device__ __forceinline__ void mfma_and_decode(const HalfCodes<kFragN> &r, const StepScales<kFragN> &sc,
                                                half8_t (&av)[kFragM], half8_t (&bv)[kFragN],
                                                floatx16 (&acc)[kFragM][kFragN]) {
  half8_t na[kFragM], nb[kFragN];
  decode_substep<kNext, kFragN>(r, sc, na, nb);
  mfma_substep<kFragN>(acc, av, bv);
  // One wavefront per SIMD issues in order, so VALU work only overlaps an
  // MFMA if it sits between MFMAs: ask for kFragM * kFragN groups of one
  // MFMA followed by a few VALU instructions.
#pragma unroll
  for (int i = 0; i < kFragM * kFragN; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kInterleave, 0);
  }
#pragma unroll
  for (int f = 0; f < kFragM; ++f) av[f] = na[f];
#pragma unroll
  for (int f = 0; f < kFragN; ++f) bv[f] = nb[f];
}

// Operand pointers and extents of one workgroup's tile.
struct TileSrc {
  const uint8_t *ac, *as, *bc, *bs;
  int64_t M, N, K, m0, n0;
};

// One K step of the pipelined main loop (K % 128 == 0).  On entry r0 holds
// the first half of this step's codes, sc_cur its scales, and av/bv the
// decoded operands of sub-step 0; stage `cur` holds this step and `nxt` the
// next one, landed or in flight.  Each sub-step's MFMAs run while the next
// sub-step is decoded.  Mid-step, one barrier makes the next step's stage
// visible (the compiler waits for this wave's global->LDS loads before it);
// then the next step's first half and scales are read into r0 and sc_nxt,
// and the step after next is fetched into `cur`, whose reads every wave has
// completed before the barrier.
template <int kFragN, bool kOff32, int kBN>
__device__ __forceinline__ void pipelined_kstep(Stage<kBN> &cur, const Stage<kBN> &nxt, const TileSrc &t, int kt,
                                                int ksteps, const LaneCoord &c, HalfCodes<kFragN> &r0,
                                                HalfCodes<kFragN> &r1, const StepScales<kFragN> &sc_cur,
                                                StepScales<kFragN> &sc_nxt, half8_t (&av)[kFragM],
                                                half8_t (&bv)[kFragN], floatx16 (&acc)[kFragM][kFragN]) {
  read_codes<kFragN>(cur, 1, c, r1);
  mfma_and_decode<1>(r0, sc_cur, av, bv, acc);
  mfma_and_decode<2>(r0, sc_cur, av, bv, acc);
  mfma_and_decode<3>(r0, sc_cur, av, bv, acc);
  mfma_and_decode<4>(r1, sc_cur, av, bv, acc);
  // This wave's global->LDS loads of the next step must have landed before
  // the barrier.  Stated explicitly: the compiler's own wait for them is not
  // reliably kept when the loads were issued in the previous loop iteration.
  // The scheduling fences pin the wait and the barrier after the MFMAs.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  read_codes<kFragN>(nxt, 0, c, r0);  // past the last step: stale but in-bounds LDS, never used
  read_scales<kFragN>(nxt, c, sc_nxt);
  if (kt + 2 < ksteps) {
    const int64_t k0 = (int64_t)(kt + 2) * BK;
    lds_load_operand<BM, kOff32>(t.ac, t.as, t.M, t.K, t.m0, k0, cur.a, cur.as);
    lds_load_operand<kBN, kOff32>(t.bc, t.bs, t.N, t.K, t.n0, k0, cur.b, cur.bs);
  }
  mfma_and_decode<5>(r1, sc_cur, av, bv, acc);
  mfma_and_decode<6>(r1, sc_cur, av, bv, acc);
  mfma_and_decode<7>(r1, sc_cur, av, bv, acc);
  mfma_and_decode<0>(r0, sc_nxt, av, bv, acc);
}

// Epilogue of one wavefront's 128 x (32 * kFragN) region at (row0, col0):
// multiply by fl(fl(sA * sB) * alpha) and store, masking the M and N edges.
// Accumulator v of lane l in a 32x32 tile holds row 8*(v/4) + 4*(l/32) + v%4,
// column l%32.
// The pipelined K step for 256 x 256 tiles, whose 256 accumulators leave
// room for one code buffer and one scale buffer only (two of each spill).
// The decoded operands are still double-buffered, so every sub-step's MFMAs
// run while the next sub-step is decoded; the cost is one exposed LDS read
// latency at each half step.  On entry r holds this step's first-half
// codes, sc its scales and av/bv sub-step 0; stage `cur` holds this step and
// `nxt` the next one, landed or in flight.
template <int kFragN, bool kOff32, int kBN>
__device__ __forceinline__ void pipelined_kstep_lite(Stage<kBN> &cur, const Stage<kBN> &nxt, const TileSrc &t, int kt,
                                                     int ksteps, const LaneCoord &c, HalfCodes<kFragN> &r,
                                                     StepScales<kFragN> &sc, half8_t (&av)[kFragM],
                                                     half8_t (&bv)[kFragN], floatx16 (&acc)[kFragM][kFragN]) {
  // Opaque copies of the lane coordinates: addresses derived from them are
  // rebuilt where used instead of being hoisted out of the loop, where they
  // would take the registers the operands need.
  LaneCoord cl = c;
  asm volatile("" : "+v"(cl.r32), "+v"(cl.h));
  mfma_and_decode<1>(r, sc, av, bv, acc);
  mfma_and_decode<2>(r, sc, av, bv, acc);
  mfma_and_decode<3>(r, sc, av, bv, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_codes<kFragN>(cur, 1, cl, r);  // the first half's codes are dead
  mfma_and_decode<4>(r, sc, av, bv, acc);
  mfma_and_decode<5>(r, sc, av, bv, acc);
  mfma_and_decode<6>(r, sc, av, bv, acc);
  mfma_and_decode<7>(r, sc, av, bv, acc);
  // Every read of `cur` is done: wait for this wave's loads of `nxt`, then
  // the barrier makes `nxt` visible and frees `cur` for the step after next.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  read_codes<kFragN>(nxt, 0, cl, r);  // past the last step: stale but in-bounds LDS, never used
  read_scales<kFragN>(nxt, cl, sc);
  if (kt + 2 < ksteps) {
    const int64_t k0 = (int64_t)(kt + 2) * BK;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    lds_load_operand<BM, kOff32>(t.ac, t.as, t.M, t.K, t.m0, k0, cur.a, cur.as, tid);
    lds_load_operand<kBN, kOff32>(t.bc, t.bs, t.N, t.K, t.n0, k0, cur.b, cur.bs, tid);
  }
  mfma_and_decode<0>(r, sc, av, bv, acc);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// The low-rank term of a LoRA-style layer ("Full-Stack FP4 ...", section
// 2.1: W = W_res + beta L2 L1, the subspace kept in BF16), folded into the
// accumulators before the main loop so that it costs no registers beside
// them: acc <- fl(q * (T L2^T)) with q = fl(beta / s), s = fl(fl(sA sB)
// alpha), and the epilogue multiplies by s, giving s acc_main + beta T L2^T
// to FP32 rounding.  With s = 0 (a zero operand, so acc_main = 0) the
// factors are q = 1 and beta.  T L2^T runs over K = lr_r on the BF16 MFMA:
// lane l takes row l % 32 of a fragment and the 8 elements at 8 (l / 32) of
// each 16-wide step, in A and B alike.  Rows and columns past the tensor
// read clamped addresses; those results are never stored.
// (q, epilogue factor) of the low-rank fold.
__device__ __forceinline__ float2 lowrank_factors(const GemmArgs &g) {
  const float s = (*g.a_st * *g.b_st) * g.alpha;
  return s != 0.0f ? make_float2(g.lr_beta / s, s) : make_float2(1.0f, g.lr_beta);
}

// The fold through LDS: per chunk of 32 along r, the workgroup copies its
// rows of T ([m0, m0 + kTM)) and of L2 ([n0, n0 + kTN)) into two LDS
// buffers (the pipeline stages, still unused), one 16-byte load per piece,
// so the chunk costs one memory latency; then each wavefront runs its
// fragments' MFMAs on operands read from LDS.  Staged rows are 80 bytes
// apart (32 BF16 and 16 bytes of padding against bank conflicts).
template <int kFragN, int kTM, int kTN, int kNT>
__device__ __forceinline__ void lowrank_init(floatx16 (&acc)[kFragM][kFragN], const GemmArgs &g, int64_t m0,
                                             int64_t n0, int wrow, int wcol, uint8_t *lt, uint8_t *ll) {
  constexpr int kPitch = 80;
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, k8 = 8 * (lane >> 5);
  for (int64_t k0 = 0; k0 < g.lr_r; k0 += 32) {
    for (int p = threadIdx.x; p < (kTM + kTN) * 4; p += kNT) {
      const bool is_t = p < kTM * 4;
      const int q = is_t ? p : p - kTM * 4;
      const int row = q >> 2, piece = q & 3;
      const int64_t kk = min(k0 + 8 * piece, g.lr_r - 8);  // past r: a repeated piece, never used
      const uint4 v = is_t ? *reinterpret_cast<const uint4 *>(g.lr_t + min(m0 + row, g.M - 1) * g.lr_r + kk)
                           : *reinterpret_cast<const uint4 *>(g.lr_l2 + min(n0 + row, g.N - 1) * g.lr_r + kk);
      *reinterpret_cast<uint4 *>((is_t ? lt : ll) + row * kPitch + 16 * piece) = v;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (k0 + 16 * u < g.lr_r) {
        bf16x8_t b[kFragN];
#pragma unroll
        for (int j = 0; j < kFragN; ++j)
          b[j] = *reinterpret_cast<const bf16x8_t *>(ll + (wcol + 32 * j + r32) * kPitch + 2 * (16 * u + k8));
#pragma unroll
        for (int i = 0; i < kFragM; ++i) {
          const bf16x8_t a =
              *reinterpret_cast<const bf16x8_t *>(lt + (wrow + 32 * i + r32) * kPitch + 2 * (16 * u + k8));
#pragma unroll
          for (int j = 0; j < kFragN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  const float q = lowrank_factors(g).x;
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j) acc[i][j] = acc[i][j] * q;
}

// Transposed epilogue staging: one 32 x 32 fragment per wave at a time, rows
// of 36 floats (16-byte aligned float4 columns, rows spread over the banks).
constexpr int kTPitch = 36;
constexpr int kTPatchBytes = 32 * kTPitch * 4;

// kRaw: store the accumulators unscaled (split-K partial tiles).
template <int kFragN, bool kBF16Out, bool kRaw = false>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[kFragM][kFragN], const GemmArgs &g, int64_t batch,
                                           int64_t wrow0, int64_t wcol0, float *tpatch) {
  using OutT = typename std::conditional<kBF16Out, uint16_t, float>::type;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r32 = lane & 31;
  const float sc = kRaw ? 1.0f : (g.lr_t ? lowrank_factors(g).y : (*g.a_st * *g.b_st) * g.alpha);
  OutT *cb_ptr = static_cast<OutT *>(g.c) + batch * g.bstride_c;
  const int64_t row0 = wrow0 + 4 * h;
  const int64_t col0 = wcol0 + r32;
  const bool full = wrow0 + 128 <= g.M && wcol0 + 32 * kFragN <= g.N;
  if constexpr (!kBF16Out) {
    if (g.staged && full) {
      // Through this wave's LDS patch, one 32 x 32 fragment at a time: the
      // fragment goes in (as its transpose when C is stored transposed) and
      // is read back by output rows, so the addend loads and the stores are
      // 16 bytes per lane, 128-byte row segments (8 rows of 32 floats per
      // instruction).  A fragment's addends are all loaded before its
      // exchange, so their latency overlaps it; each lane reads exactly the
      // addends of the elements it stores, so c may be the output itself.
      // Only this wave uses the patch and its LDS accesses run in order; the
      // fences keep the compiler from moving them across each other.
      // y = fl(fl(acc * s) + fl(beta * c)) as below.
      const float *ci_ptr = g.cin ? g.cin + batch * g.bstride_cin : nullptr;
      const int prow = lane >> 3, pcol = 4 * (lane & 7);
#pragma unroll
      for (int i = 0; i < kFragM; ++i) {
#pragma unroll
        for (int j = 0; j < kFragN; ++j) {
          // the lane's first output element of this fragment
          const int64_t orow = g.ct ? wcol0 + 32 * j + prow : wrow0 + 32 * i + prow;
          const int64_t ocol = g.ct ? wrow0 + 32 * i + pcol : wcol0 + 32 * j + pcol;
          float4 cv[4];
          if (ci_ptr) {
#pragma unroll
            for (int p = 0; p < 4; ++p) cv[p] = *reinterpret_cast<const float4 *>(ci_ptr + (orow + 8 * p) * g.ldcin + ocol);
          }
          if (g.ct) {
            // accumulator rows 8q + 4h + t (t = 0..3) of column r32 -> patch row r32
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4 *>(tpatch + r32 * kTPitch + 8 * q + 4 * h) =
                  make_float4(acc[i][j][4 * q] * sc, acc[i][j][4 * q + 1] * sc, acc[i][j][4 * q + 2] * sc,
                              acc[i][j][4 * q + 3] * sc);
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) tpatch[(8 * (v >> 2) + 4 * h + (v & 3)) * kTPitch + r32] = acc[i][j][v] * sc;
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            float4 y = *reinterpret_cast<const float4 *>(tpatch + (prow + 8 * p) * kTPitch + pcol);
            if (ci_ptr) {
              y.x += g.beta * cv[p].x;
              y.y += g.beta * cv[p].y;
              y.z += g.beta * cv[p].z;
              y.w += g.beta * cv[p].w;
            }
            *reinterpret_cast<float4 *>(cb_ptr + (orow + 8 * p) * g.ldc + ocol) = y;
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        }
      }
      return;
    }
    if (g.ct) {
      // Transposed store of a partial tile, element by element (element
      // (r, c) at c * ldc + r); y = fl(fl(acc * s) + fl(beta * c)) as below.
      const float *ci_ptr = g.cin ? g.cin + batch * g.bstride_cin : nullptr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int i = 0; i < kFragM; ++i) {
          const int64_t r = row0 + 8 * q + 32 * i;
#pragma unroll
          for (int j = 0; j < kFragN; ++j) {
            const int64_t col = col0 + 32 * j;
            if (col >= g.N) continue;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              if (r + t >= g.M) continue;
              float y = acc[i][j][4 * q + t] * sc;
              if (ci_ptr) y += g.beta * ci_ptr[col * g.ldcin + r + t];
              cb_ptr[col * g.ldc + r + t] = y;
            }
          }
        }
      }
      return;
    }
  }
  if (g.cin) {
    // y = fl(fl(acc * s) + fl(beta * c)): each element is read and written
    // by the same lane, so c may be the output itself.  The addends of one
    // accumulator row pair of one fragment row are loaded before any is used
    // (addresses clamped into the tensor, so the loads need no predicate and
    // issue back to back).
    const float *ci_ptr = g.cin + batch * g.bstride_cin;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const int64_t rv = row0 + 8 * (v >> 2) + (v & 3);
#pragma unroll
      for (int i = 0; i < kFragM; ++i) {
        const int64_t r = rv + 32 * i;
        const int64_t r0 = min(r, g.M - 1), r1 = min(r + 1, g.M - 1);
        float cv[kFragN][2];
#pragma unroll
        for (int j = 0; j < kFragN; ++j) {
          const int64_t col = min(col0 + 32 * j, g.N - 1);
          cv[j][0] = ci_ptr[r0 * g.ldcin + col];
          cv[j][1] = ci_ptr[r1 * g.ldcin + col];
        }
#pragma unroll
        for (int j = 0; j < kFragN; ++j) {
          const int64_t col = col0 + 32 * j;
          const bool col_ok = full || col < g.N;
          const bool ok0 = col_ok && (full || r < g.M), ok1 = col_ok && (full || r + 1 < g.M);
          const float y0 = acc[i][j][v] * sc + g.beta * cv[j][0];
          const float y1 = acc[i][j][v + 1] * sc + g.beta * cv[j][1];
          OutT *pr = cb_ptr + r * g.ldc + col;
          if constexpr (kBF16Out) {
            const uint32_t b2 = pack_bf16x2_rne(y0, y1);
            if (ok0) pr[0] = (uint16_t)b2;
            if (ok1) pr[g.ldc] = (uint16_t)(b2 >> 16);
          } else {
            if (ok0) pr[0] = y0;
            if (ok1) pr[g.ldc] = y1;
          }
        }
      }
    }
    return;
  }
  // One accumulator row pair at a time, so no table of row offsets stays
  // live beside the accumulators.
#pragma unroll
  for (int v = 0; v < 16; v += 2) {
    const int64_t rv = row0 + 8 * (v >> 2) + (v & 3);
    OutT *p0 = cb_ptr + rv * g.ldc + col0;
#pragma unroll
    for (int i = 0; i < kFragM; ++i) {
      const int64_t r = rv + 32 * i;
      OutT *pr = p0 + 32 * i * g.ldc;
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const bool col_ok = full || col0 + 32 * j < g.N;
        const bool ok0 = col_ok && (full || r < g.M), ok1 = col_ok && (full || r + 1 < g.M);
        if constexpr (kBF16Out) {
          // v_cvt_pk_bf16_f32: two FP32 -> BF16, round to nearest even
          const uint32_t b2 = pack_bf16x2_rne(acc[i][j][v] * sc, acc[i][j][v + 1] * sc);
          if (ok0) pr[32 * j] = (uint16_t)b2;
          if (ok1) pr[g.ldc + 32 * j] = (uint16_t)(b2 >> 16);
        } else {
          if (ok0) pr[32 * j] = acc[i][j][v] * sc;
          if (ok1) pr[g.ldc + 32 * j] = acc[i][j][v + 1] * sc;
        }
      }
    }
  }
}

// kSym: one (tile pair, K range) item of a symmetric product split along K
// (the upper-triangle tile (I, J), I <= J, over K steps [split * sym_steps,
// ...)), stored unscaled as a partial tile; sym_reduce_kernel finishes it.
template <int kFragN, bool kFast, bool kBF16Out, bool kOff32, bool kSym = false>
__global__ __launch_bounds__(kThreads) void gemm_nvfp4_kernel(GemmArgs g) {
  constexpr int kBN = 64 * kFragN;
  static_assert(!kSym || (kFragN == 4 && kFast && !kBF16Out), "split-K items are square FP32 tiles");
  // Two stages as separate objects: the compiler can then tell a read of one
  // from a global->LDS load in flight into the other and does not wait for it.
  __shared__ Stage<kBN> st0, st1;

  int tm, tn;
  int64_t kbeg = 0;  // first K element of this item
  int ksteps = (int)((g.K + BK - 1) / BK);
  if constexpr (kSym) {
    const int pair = (int)blockIdx.x / g.sym_splits, split = (int)blockIdx.x - pair * g.sym_splits;
    int row = 0, rem = pair;  // row-major upper triangle: row I holds T - I pairs
    while (rem >= g.sym_t - row) {
      rem -= g.sym_t - row;
      ++row;
    }
    tm = row;
    tn = row + rem;
    kbeg = (int64_t)split * g.sym_steps * BK;
    ksteps = min(g.sym_steps, ksteps - split * g.sym_steps);
  } else {
    // XCD-aware tile order: consecutive workgroups go to different XCDs, so
    // give XCD x the x-th contiguous slice of the grouped tile order.  Groups
    // of kGroup tile rows: 8 for the square tile, 4 where the A tile is the
    // larger (an XCD's 32 concurrent tiles then span 4 x 8 of them, the
    // least operand data per XCD).
    constexpr int kGroup = kFragN == 4 ? kGroupM : 4;
    const int ntiles = g.tiles_m * g.tiles_n;
    const int bid = blockIdx.x;
    const int per_xcd = ntiles / 8;
    const int t = (ntiles % 8 == 0) ? (bid % 8) * per_xcd + bid / 8 : bid;
    const int group = t / (kGroup * g.tiles_n);
    const int first_m = group * kGroup;
    const int gm = min(g.tiles_m - first_m, kGroup);
    const int in_group = t - group * kGroup * g.tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
  }

  const int64_t batch = blockIdx.y;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * kBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  // (K stays the row stride; a split item starts kbeg elements in)
  const uint8_t *ac = g.a_codes + batch * g.M * (g.K / 2) + kbeg / 2;
  const uint8_t *as = g.a_scales + batch * g.M * (g.K / 16) + kbeg / 16;
  const uint8_t *bc = g.b_codes + batch * g.N * (g.K / 2) + kbeg / 2;
  const uint8_t *bs = g.b_scales + batch * g.N * (g.K / 16) + kbeg / 16;

  floatx16 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  // (the 256 x 256 tile has no registers to spare for it: never chosen with
  // the low-rank term)
  if constexpr (kFragN < 4) {
    static_assert(BM * 80 <= sizeof(Stage<kBN>) && kBN * 80 <= sizeof(Stage<kBN>), "low-rank staging fits a stage");
    if (g.lr_t)
      lowrank_init<kFragN, BM, kBN, kThreads>(acc, g, m0, n0, wm * 128, wn * (32 * kFragN),
                                              reinterpret_cast<uint8_t *>(&st0), reinterpret_cast<uint8_t *>(&st1));
  }

  if constexpr (kFast && kFragN <= 3) {
    const TileSrc src{ac, as, bc, bs, g.M, g.N, g.K, m0, n0};
    const LaneCoord c{wm, wn, h, r32};
    if (ksteps > 0) {
      lds_load_operand<BM, kOff32>(ac, as, g.M, g.K, m0, 0, st0.a, st0.as);
      lds_load_operand<kBN, kOff32>(bc, bs, g.N, g.K, n0, 0, st0.b, st0.bs);
      if (ksteps > 1) {
        lds_load_operand<BM, kOff32>(ac, as, g.M, g.K, m0, BK, st1.a, st1.as);
        lds_load_operand<kBN, kOff32>(bc, bs, g.N, g.K, n0, BK, st1.b, st1.bs);
      }
    }
    // Stage loads issued as assembly are not seen by the compiler's own
    // wait before a barrier: wait for them explicitly.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    HalfCodes<kFragN> r0, r1;
    StepScales<kFragN> sc0, sc1;  // scales of even / odd steps
    half8_t av[kFragM], bv[kFragN];
    read_codes<kFragN>(st0, 0, c, r0);
    read_scales<kFragN>(st0, c, sc0);
    decode_substep<0, kFragN>(r0, sc0, av, bv);
    for (int kt = 0; kt < ksteps; kt += 2) {
      pipelined_kstep<kFragN, kOff32>(st0, st1, src, kt, ksteps, c, r0, r1, sc0, sc1, av, bv, acc);
      if (kt + 1 < ksteps) pipelined_kstep<kFragN, kOff32>(st1, st0, src, kt + 1, ksteps, c, r0, r1, sc1, sc0, av, bv, acc);
    }
  } else if constexpr (kFast) {
    const TileSrc src{ac, as, bc, bs, g.M, g.N, g.K, m0, n0};
    const LaneCoord c{wm, wn, h, r32};
    if (ksteps > 0) {
      lds_load_operand<BM, kOff32>(ac, as, g.M, g.K, m0, 0, st0.a, st0.as);
      lds_load_operand<kBN, kOff32>(bc, bs, g.N, g.K, n0, 0, st0.b, st0.bs);
      if (ksteps > 1) {
        lds_load_operand<BM, kOff32>(ac, as, g.M, g.K, m0, BK, st1.a, st1.as);
        lds_load_operand<kBN, kOff32>(bc, bs, g.N, g.K, n0, BK, st1.b, st1.bs);
      }
    }
    // Stage loads issued as assembly are not seen by the compiler's own
    // wait before a barrier: wait for them explicitly.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    HalfCodes<kFragN> r;
    StepScales<kFragN> sc;
    half8_t av[kFragM], bv[kFragN];
    read_codes<kFragN>(st0, 0, c, r);
    read_scales<kFragN>(st0, c, sc);
    decode_substep<0, kFragN>(r, sc, av, bv);
    for (int kt = 0; kt < ksteps; kt += 2) {
      pipelined_kstep_lite<kFragN, kOff32>(st0, st1, src, kt, ksteps, c, r, sc, av, bv, acc);
      if (kt + 1 < ksteps) pipelined_kstep_lite<kFragN, kOff32>(st1, st0, src, kt + 1, ksteps, c, r, sc, av, bv, acc);
    }
  } else {
    StagedLoad<BM> la;
    StagedLoad<kBN> lb;
    if (ksteps > 0) {
      la.load(ac, as, g.M, g.K, m0, 0);
      lb.load(bc, bs, g.N, g.K, n0, 0);
      la.store(st0.a, st0.as);
      lb.store(st0.b, st0.bs);
    }
    __syncthreads();
    for (int kt = 0; kt < ksteps; ++kt) {
      const Stage<kBN> &cur = (kt & 1) ? st1 : st0;
      Stage<kBN> &nxt = (kt & 1) ? st0 : st1;
      const bool more = kt + 1 < ksteps;
      // This lane's 32 code bytes and 4 scale bytes of every fragment.
      uint4 ca[kFragM][2], cb[kFragN][2];
      half2_t sa[kFragM][2], sb[kFragN][2];
#pragma unroll
      for (int f = 0; f < kFragM; ++f) {
        const int r = wm * 128 + f * 32 + r32;
        ca[f][0] = *reinterpret_cast<const uint4 *>(cur.a + 16 * chunk_slot(r, 2 * h));
        ca[f][1] = *reinterpret_cast<const uint4 *>(cur.a + 16 * chunk_slot(r, 2 * h + 1));
        const uint32_t w = h ? cur.as[r].y : cur.as[r].x;
        sa[f][0] = scale_pair_lo(w);
        sa[f][1] = scale_pair_lo(w >> 16);
      }
#pragma unroll
      for (int f = 0; f < kFragN; ++f) {
        const int r = wn * (32 * kFragN) + f * 32 + r32;
        cb[f][0] = *reinterpret_cast<const uint4 *>(cur.b + 16 * chunk_slot(r, 2 * h));
        cb[f][1] = *reinterpret_cast<const uint4 *>(cur.b + 16 * chunk_slot(r, 2 * h + 1));
        const uint32_t w = h ? cur.bs[r].y : cur.bs[r].x;
        sb[f][0] = scale_pair_lo(w);
        sb[f][1] = scale_pair_lo(w >> 16);
      }
      if (more) {
        la.load(ac, as, g.M, g.K, m0, (int64_t)(kt + 1) * BK);
        lb.load(bc, bs, g.N, g.K, n0, (int64_t)(kt + 1) * BK);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        half8_t av[kFragM], bv[kFragN];
#pragma unroll
        for (int f = 0; f < kFragM; ++f) av[f] = decode8_s256(word_of(ca[f][s >> 2], s & 3), sa[f][s >> 2][(s >> 1) & 1]);
#pragma unroll
        for (int f = 0; f < kFragN; ++f) bv[f] = decode8_s256(word_of(cb[f][s >> 2], s & 3), sb[f][s >> 2][(s >> 1) & 1]);
        mfma_substep<kFragN>(acc, av, bv);
      }
      if (more) {
        la.store(nxt.a, nxt.as);
        lb.store(nxt.b, nxt.bs);
      }
      __syncthreads();
    }
  }

  // The stages are free for the staged epilogue (an addend, C transposed, or
  // a partial tile): every wave has passed the main loop's last barrier, no
  // global->LDS load is in flight, and what a wave still reads from the
  // stages after that barrier is never used.
  static_assert(4 * kTPatchBytes <= sizeof(Stage<kBN>), "transpose patches fit a stage");
  float *patch = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(&st0) + wave * kTPatchBytes);
  if constexpr (kSym) {
    // the partial tile, unscaled, [BM][BM] row-major
    GemmArgs gp = g;
    gp.c = g.sym_part + (int64_t)blockIdx.x * (BM * kBN);
    gp.M = BM;
    gp.N = kBN;
    gp.ldc = kBN;
    gp.bstride_c = 0;
    gp.cin = nullptr;
    gp.lr_t = nullptr;
    gp.ct = false;
    gp.staged = true;
    store_tile<kFragN, false, true>(acc, gp, 0, wm * 128, wn * (32 * kFragN), patch);
  } else {
    store_tile<kFragN, kBF16Out>(acc, g, batch, m0 + wm * 128, n0 + wn * (32 * kFragN), patch);
  }
}

// ---------------------------------------------------------------------------
// Two wavefronts per SIMD.  A workgroup of 8 wavefronts computes a
// (128 kWM) x (96 kWN) tile; each wavefront still owns a 128 x 96 region
// (4 x 3 MFMA tiles), so the decode work per MFMA is that of the 256 x 192
// kernel above.  With two wavefronts on every SIMD, one wavefront's decode
// and LDS reads issue while the other's MFMAs run, and a wavefront waiting
// at the step barrier or for an LDS read leaves the matrix pipe to the
// other.  The 192 accumulators leave 64 registers per wavefront for
// everything else, so a step holds little: the scale words of its seven
// fragments, then per half step the seven scale pairs, per two sub-steps
// the seven code words, the three B operands and one A operand.
//
// Three LDS stages: the global->LDS loads of step k + 2 are issued right
// after the barrier that opens step k, into the stage step k - 1 used, and
// each wavefront waits only for its own loads of step k (those of step
// k + 1, issued later, stay in flight).
// ---------------------------------------------------------------------------
constexpr int kW8Threads = 512;

template <int kBM, int kBN>
struct alignas(16) W8Stage {
  uint8_t a[kBM * kRowBytes];
  uint8_t b[kBN * kRowBytes];
  uint2 as[kBM];
  uint2 bs[kBN];
};

// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt left at their maxima.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// The global->LDS loads of one stage, split into jobs of one instruction:
// code jobs move 16 rows (1 KB, 16 bytes per lane), scale jobs 32 rows
// (256 B, one dword per lane).  Jobs are numbered A codes, A scales, B codes,
// B scales, and job j belongs to wavefront j mod 8, so a wavefront's i-th job
// has a kind known at compile time unless its group of eight straddles a
// kind boundary.  A lane's global offset is recomputed at every issue (rows
// clamped to the last row, code chunks unswizzled): holding it across the
// step would cost registers the accumulators need.  Offsets are 32-bit; the
// launcher only picks this kernel for operands under 2 GiB.
template <int kWM, int kWN>
struct W8Loader {
  static constexpr int kBM = 128 * kWM, kBN = 96 * kWN;
  static constexpr int kCodeA = kBM / 16, kScaleA = kBM / 32, kCodeB = kBN / 16, kScaleB = kBN / 32;
  static constexpr int kJobs = kCodeA + kScaleA + kCodeB + kScaleB;
  static constexpr int kPerWave = (kJobs + 7) / 8;
  static_assert(kBM % 32 == 0 && kBN % 32 == 0, "scale jobs cover 32 rows of one operand");
  static_assert(sizeof(W8Stage<kBM, kBN>) == (kBM + kBN) * (kRowBytes + 8), "stage members are packed");

  const uint8_t *ac, *as, *bc, *bs;
  int64_t M, N, m0, n0;
  uint32_t kb2, kb16;  // bytes per code row, per scale row

  // Byte offsets of the stage members (W8Stage has no padding between them).
  static constexpr uint32_t kOffB = kBM * kRowBytes, kOffAs = (kBM + kBN) * kRowBytes,
                            kOffBs = kOffAs + kBM * 8;

  // kind 0: A codes, 1: A scales, 2: B codes, 3: B scales; jj: job within its
  // kind; sbase: the stage's LDS address (scalar).  Lane terms shared by all
  // jobs of a kind: a code job's lane takes row 16 jj + lane / 4 and, since
  // 16 jj leaves row bits 2..3 alone, the same unswizzled chunk; a scale
  // job's lane takes row 32 jj + lane / 2, dword lane & 1.  Rows are clamped
  // to the last row; all of it in 32 bits (operands under 2 GiB, fewer than
  // 2^24 rows and code bytes per row, which the launcher checks).
  struct LaneTerms {
    int code_row, code_off, scale_row, scale_off;
  };
  __device__ __forceinline__ static LaneTerms lane_terms(int lane) {
    const int code_row = lane >> 2;
    return LaneTerms{code_row, 16 * (chunk_slot(code_row, lane & 3) & 3), lane >> 1, 4 * (lane & 1)};
  }

  template <int kKind>
  __device__ __forceinline__ void job(uint32_t sbase, int jj, const LaneTerms &t, int64_t k0) const {
    if constexpr (kKind == 0 || kKind == 2) {
      const int last = (int)(kKind == 0 ? M - 1 - m0 : N - 1 - n0);  // last row relative to the tile
      const uint32_t r0 = (uint32_t)(kKind == 0 ? m0 : n0);
      const uint32_t gr = r0 + (uint32_t)min(16 * jj + t.code_row, last);
      dma<16>((kKind == 0 ? ac : bc) + k0 / 2, __umul24(gr, kb2) + (uint32_t)t.code_off,
              sbase + (kKind == 0 ? 0u : kOffB) + 1024u * jj);
    } else {
      const int last = (int)(kKind == 1 ? M - 1 - m0 : N - 1 - n0);
      const uint32_t r0 = (uint32_t)(kKind == 1 ? m0 : n0);
      const uint32_t gr = r0 + (uint32_t)min(32 * jj + t.scale_row, last);
      dma<4>((kKind == 1 ? as : bs) + k0 / 16, __umul24(gr, kb16) + (uint32_t)t.scale_off,
             sbase + (kKind == 1 ? kOffAs : kOffBs) + 256u * jj);
    }
  }

  template <int kI>
  __device__ __forceinline__ void issue_one(uint32_t st, int wave, const LaneTerms &lane, int64_t k0) const {
    constexpr int lo = 8 * kI, hi = 8 * kI + 7;
    constexpr int e0 = kCodeA, e1 = e0 + kScaleA, e2 = e1 + kCodeB, e3 = e2 + kScaleB;
    const int j = lo + wave;
    if constexpr (hi < e0) {
      job<0>(st, j, lane, k0);
    } else if constexpr (lo >= e0 && hi < e1) {
      job<1>(st, j - e0, lane, k0);
    } else if constexpr (lo >= e1 && hi < e2) {
      job<2>(st, j - e1, lane, k0);
    } else if constexpr (lo >= e2 && hi < e3) {
      job<3>(st, j - e2, lane, k0);
    } else {  // the group straddles a kind boundary: branch on the (uniform) job index
      if (j < e0) job<0>(st, j, lane, k0);
      else if (j < e1) job<1>(st, j - e0, lane, k0);
      else if (j < e2) job<2>(st, j - e1, lane, k0);
      else if (j < e3) job<3>(st, j - e2, lane, k0);
    }
  }

  template <int... kIs>
  __device__ __forceinline__ void issue_all(uint32_t st, int wave, const LaneTerms &lane, int64_t k0,
                                            std::integer_sequence<int, kIs...>) const {
    (issue_one<kIs>(st, wave, lane, k0), ...);
  }

  __device__ __forceinline__ void issue(W8Stage<kBM, kBN> &st, int wave, int lane, int64_t k0) const {
    const uint32_t sbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&st);
    const LaneTerms t = lane_terms(lane);
    issue_all(sbase, wave, t, k0, std::make_integer_sequence<int, kPerWave>{});
  }

  // Wait until this wavefront's loads of the oldest stage in flight have
  // landed while the next stage's (issued after them) stay in flight.  Any
  // other vector-memory operation issued later only makes the wait stricter.
  __device__ __forceinline__ static void wait_oldest(int wave) {
    constexpr int kFull = kJobs / 8, kRem = kJobs % 8;  // wavefronts < kRem issue one more job
    __builtin_amdgcn_sched_barrier(0);
    if (kRem != 0 && wave < kRem)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kFull + 1));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kFull));
    __builtin_amdgcn_sched_barrier(0);
  }
};

// The MFMAs of one K step for one wavefront's 128 x 96 region.
template <int kBM, int kBN>
__device__ __forceinline__ void w8_compute(const W8Stage<kBM, kBN> &st, int arow, int brow, int h, int qa, int qb,
                                           floatx16 (&acc)[kFragM][3]) {
  const uint32_t *as32 = reinterpret_cast<const uint32_t *>(st.as);
  const uint32_t *bs32 = reinterpret_cast<const uint32_t *>(st.bs);
  uint32_t wa[kFragM], wb[3];
#pragma unroll
  for (int f = 0; f < kFragM; ++f) wa[f] = as32[(arow + 32 * f) * 2 + h];
#pragma unroll
  for (int f = 0; f < 3; ++f) wb[f] = bs32[(brow + 32 * f) * 2 + h];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // blocks 4h + 2 half (low) and 4h + 2 half + 1 (high) of every fragment
    half2_t sa[kFragM], sb[3];
#pragma unroll
    for (int f = 0; f < kFragM; ++f) sa[f] = scale_pair_lo(wa[f] >> (16 * half));
#pragma unroll
    for (int f = 0; f < 3; ++f) sb[f] = scale_pair_lo(wb[f] >> (16 * half));
    const int ca_off = 16 * ((2 * h + half) ^ qa), cb_off = 16 * ((2 * h + half) ^ qb);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint2 ca[kFragM], cb[3];
#pragma unroll
      for (int f = 0; f < kFragM; ++f)
        ca[f] = *reinterpret_cast<const uint2 *>(st.a + (arow + 32 * f) * kRowBytes + ca_off + 8 * p);
#pragma unroll
      for (int f = 0; f < 3; ++f)
        cb[f] = *reinterpret_cast<const uint2 *>(st.b + (brow + 32 * f) * kRowBytes + cb_off + 8 * p);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        half8_t bv[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) bv[j] = decode8_s256(e ? cb[j].y : cb[j].x, sb[j][p]);
#pragma unroll
        for (int i = 0; i < kFragM; ++i) {
          const half8_t av = decode8_s256(e ? ca[i].y : ca[i].x, sa[i][p]);
#pragma unroll
          for (int j = 0; j < 3; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv[j], acc[i][j], 0, 0, 0);
        }
      }
      // Keep the scheduler from hoisting later sub-steps' reads and decodes
      // into this one: the other wavefront on the SIMD hides the latency,
      // and the registers are not there.
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

struct W8Lane {
  int wave, lane, h, arow, brow, qa, qb;
};

// Fill a stage with K step `kstep`.  The stage comes in as a restrict
// pointer so that, once inlined, its loads carry alias-scope information: the
// compiler then tells them apart from reads of the other stages instead of
// waiting for every load that writes LDS before any LDS read.
template <int kWM, int kWN>
__device__ __forceinline__ void w8_fill(W8Stage<128 * kWM, 96 * kWN> *__restrict__ dst, const W8Loader<kWM, kWN> &ld,
                                        const W8Lane &c, int kstep) {
  // Offsets are recomputed per issue; an opaque copy of the lane index keeps
  // them from being hoisted out of the loop (and spilled).
  int lane_k = c.lane;
  asm volatile("" : "+v"(lane_k));
  ld.issue(*dst, c.wave, lane_k, (int64_t)kstep * BK);
}

// One K step: wait for this step's stage, barrier, refill the stage the step
// before used, multiply.  The refill is issued at every step, for step
// kt + 2 or, past the end, again for the last step (into a stage nobody reads
// any more): a fixed number of loads per step lets the compiler's own wait
// before the reads of `cur` be exact instead of draining every load.
template <int kWM, int kWN>
__device__ __forceinline__ void w8_step(const W8Stage<128 * kWM, 96 * kWN> *__restrict__ cur,
                                        W8Stage<128 * kWM, 96 * kWN> *__restrict__ dst,
                                        const W8Loader<kWM, kWN> &ld, const W8Lane &c, int kt, int ksteps,
                                        floatx16 (&acc)[kFragM][3]) {
  W8Loader<kWM, kWN>::wait_oldest(c.wave);
  // A bare barrier: __syncthreads() would also wait for the loads of the
  // next stage, still in flight.  This wavefront's LDS reads of the step
  // before have all returned (lgkmcnt(0)) before it arrives, so the stage
  // they read can be refilled once every wavefront has arrived.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  w8_fill<kWM, kWN>(dst, ld, c, min(kt + 2, ksteps - 1));
  __builtin_amdgcn_sched_barrier(0);
  w8_compute<128 * kWM, 96 * kWN>(*cur, c.arow, c.brow, c.h, c.qa, c.qb, acc);
}

template <int kWM, int kWN, bool kBF16Out, bool kLowRank>
__global__ __launch_bounds__(kW8Threads) void gemm_nvfp4_w8_kernel(GemmArgs g) {
  using L = W8Loader<kWM, kWN>;
  constexpr int kBM = L::kBM, kBN = L::kBN;
  // Three stages as separate objects, so the compiler can tell reads of one
  // from the global->LDS loads in flight into the others.
  __shared__ W8Stage<kBM, kBN> st0, st1, st2;

  // XCD-aware grouped order as in the 4-wavefront kernel; with the tall
  // 512 x 192 tile (A tiles 2.7 times the B tiles), groups of 4 tile rows
  // give an XCD's 32 concurrent tiles a 4 x 8 block, the least operand data
  // per XCD: 51 MB fetched at 8192 x 3072 x 3072 against 70 MB with 8 x 4.
  constexpr int kGroup = kBM > kBN ? 4 : kGroupM;
  const int ntiles = g.tiles_m * g.tiles_n;
  const int bid = blockIdx.x;
  const int per_xcd = ntiles / 8;
  const int t = (ntiles % 8 == 0) ? (bid % 8) * per_xcd + bid / 8 : bid;
  const int group = t / (kGroup * g.tiles_n);
  const int first_m = group * kGroup;
  const int gm = min(g.tiles_m - first_m, kGroup);
  const int in_group = t - group * kGroup * g.tiles_n;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;

  const int64_t batch = blockIdx.y;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  const int h = lane >> 5, r32 = lane & 31;
  const int arow = wm * 128 + r32, brow = wn * 96 + r32;
  // The chunk swizzle of the lane's rows (the same for rows 32 apart).
  const int qa = chunk_slot(arow, 0) & 3, qb = chunk_slot(brow, 0) & 3;

  const uint8_t *ac = g.a_codes + batch * g.M * (g.K / 2);
  const uint8_t *as = g.a_scales + batch * g.M * (g.K / 16);
  const uint8_t *bc = g.b_codes + batch * g.N * (g.K / 2);
  const uint8_t *bs = g.b_scales + batch * g.N * (g.K / 16);

  floatx16 acc[kFragM][3];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  // a separate instantiation: the kernel runs at its register limit
  if constexpr (kLowRank) {
    static_assert(kBM * 80 <= sizeof(W8Stage<kBM, kBN>) && kBN * 80 <= sizeof(W8Stage<kBM, kBN>),
                  "low-rank staging fits a stage");
    lowrank_init<3, kBM, kBN, kW8Threads>(acc, g, m0, n0, wm * 128, wn * 96, reinterpret_cast<uint8_t *>(&st0),
                                          reinterpret_cast<uint8_t *>(&st1));
  }

  const L ld{ac, as, bc, bs, g.M, g.N, m0, n0, (uint32_t)(g.K / 2), (uint32_t)(g.K / 16)};
  const int ksteps = (int)(g.K / BK);
  const W8Lane c{wave, lane, h, arow, brow, qa, qb};
  if (ksteps > 0) {  // steps 0 and 1 (or the last step again): one stage in flight per step from here on
    w8_fill<kWM, kWN>(&st0, ld, c, 0);
    w8_fill<kWM, kWN>(&st1, ld, c, min(1, ksteps - 1));
  }
  for (int kt = 0; kt < ksteps; kt += 3) {
    w8_step<kWM, kWN>(&st0, &st2, ld, c, kt, ksteps, acc);
    if (kt + 1 < ksteps) w8_step<kWM, kWN>(&st1, &st0, ld, c, kt + 1, ksteps, acc);
    if (kt + 2 < ksteps) w8_step<kWM, kWN>(&st2, &st1, ld, c, kt + 2, ksteps, acc);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the refills issued past the last step
  // The staged epilogue (an addend, or C transposed) uses st0 once every
  // wave is done with the stages.
  static_assert(8 * kTPatchBytes <= sizeof(W8Stage<kBM, kBN>), "transpose patches fit a stage");
  if (g.staged) __syncthreads();
  store_tile<3, kBF16Out>(acc, g, batch, m0 + wm * 128, n0 + wn * 96,
                          reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(&st0) + wave * kTPatchBytes));
}

template <int kFragN>
hipError_t launch_tiles(const GemmArgs &g, int64_t batch, bool fast, bool bf16, bool off32, hipStream_t s) {
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n), (unsigned)batch);
  const dim3 block(kThreads);
  if (fast && off32) {
    if (bf16) hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, true, true, true>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, true, false, true>), grid, block, 0, s, g);
  } else if (fast) {
    if (bf16) hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, true, true, false>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, true, false, false>), grid, block, 0, s, g);
  } else if (bf16) {
    hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, false, true, false>), grid, block, 0, s, g);
  } else {
    hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, false, false, false>), grid, block, 0, s, g);
  }
  return hipGetLastError();
}

template <int kWM, int kWN>
hipError_t launch_w8(const GemmArgs &g, int64_t batch, bool bf16, hipStream_t s) {
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n), (unsigned)batch);
  if (g.lr_t) {
    if (bf16) hipLaunchKernelGGL((gemm_nvfp4_w8_kernel<kWM, kWN, true, true>), grid, dim3(kW8Threads), 0, s, g);
    else hipLaunchKernelGGL((gemm_nvfp4_w8_kernel<kWM, kWN, false, true>), grid, dim3(kW8Threads), 0, s, g);
  } else if (bf16) {
    hipLaunchKernelGGL((gemm_nvfp4_w8_kernel<kWM, kWN, true, false>), grid, dim3(kW8Threads), 0, s, g);
  } else {
    hipLaunchKernelGGL((gemm_nvfp4_w8_kernel<kWM, kWN, false, false>), grid, dim3(kW8Threads), 0, s, g);
  }
  return hipGetLastError();
}

// Kernel and tile choice.  Candidates: the 4-wavefront kernel with 256 x 256,
// 256 x 192 and 256 x 128 tiles, and (K % 128 == 0) the 8-wavefront kernel
// with 512 x 192 and 256 x 384 tiles.  Each is costed as its rounds of
// workgroups (one workgroup per CU, 256 CUs; a partly filled last round
// counts in full) times its tile area times a per-element cost measured on
// fprop/MLP-sized problems.
struct TilePick {
  int kind;  // 4-wavefront kFragN (4, 3, 2), or 8-wavefront: 10 (512 x 192), 11 (256 x 384)
  int bm, bn;
  double cost;  // rounds of 256 tiles x tile area x the kernel's relative cost per element
};

// The 8-wavefront kernels need K % BK == 0; their loads use 32-bit offsets
// within an operand and 24-bit row and row-size factors.
bool w8_applies(int64_t M, int64_t N, int64_t K) {
  return K % BK == 0 && M * (K / 2) < ((int64_t)1 << 31) && N * (K / 2) < ((int64_t)1 << 31) && M < (1 << 24) &&
         N < (1 << 24) && K / 2 < (1 << 24);
}

TilePick pick_tiles(int64_t M, int64_t N, int64_t batch, bool fast, int force_bm, int force_bn, bool lowrank) {
  struct Cand {
    int kind, bm, bn;
    double cost;
    bool need_fast;
  };
  const Cand cands[5] = {{10, 512, 192, 0.96, true}, {11, 256, 384, 0.96, true},
                         {4, 256, 256, 1.0, false},  {3, 256, 192, 1.02, false}, {2, 256, 128, 1.12, false}};
  double best = 1e300;
  TilePick pick{4, 256, 256, 0.0};
  for (const Cand &c : cands) {
    if (c.need_fast && !fast) continue;
    if (lowrank && c.kind == 4) continue;
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * batch;
    const double t = (double)((tiles + 255) / 256) * c.bm * c.bn * c.cost;
    if (t < best - 1e-9) {
      best = t;
      pick = TilePick{c.kind, c.bm, c.bn, t};
    }
  }
  // A requested tile (tuning and tests) replaces the choice where its
  // kernel applies; otherwise the request is refused.
  if (force_bm != 0 || force_bn != 0) {
    pick = TilePick{-1, 0, 0, 0.0};
    for (const Cand &c : cands)
      if (c.bm == force_bm && c.bn == force_bn && (fast || !c.need_fast) && !(lowrank && c.kind == 4))
        pick = TilePick{c.kind, c.bm, c.bn, 0.0};
  }
  return pick;
}

// Finish a symmetric split-K product: for tile pair (I, J) and a 64 x 64
// sub-block of it, add the partial tiles in split order, y = fl(fl(sum * s) +
// fl(beta * c)) at (r, c), and when I != J the same sums at the mirrored
// position (c, r) with that position's addend (the sums go through LDS to be
// read back by the mirror's rows).
struct SymArgs {
  const float *part;
  int T, S;
  int64_t m;
  const float *a_st, *b_st;
  float alpha;
  const float *cin;  // optional [m][m], row stride ldcin
  int64_t ldcin;
  float beta;
  float *c;  // [m][m], row stride ldc
  int64_t ldc;
};

__global__ __launch_bounds__(256) void sym_reduce_kernel(SymArgs a) {
  __shared__ float tr[64][65];
  const int pair = (int)blockIdx.x >> 4, sub = (int)blockIdx.x & 15;
  int I = 0, rem = pair;
  while (rem >= a.T - I) {
    rem -= a.T - I;
    ++I;
  }
  const int J = I + rem;
  const int sr = sub >> 2, sc4 = sub & 3;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const float s = (*a.a_st * *a.b_st) * a.alpha;
  const int64_t R0 = (int64_t)I * BM + 64 * sr, C0 = (int64_t)J * BM + 64 * sc4;
  const float *p0 = a.part + (int64_t)pair * a.S * (BM * BM) + (64 * sr) * BM + 64 * sc4 + 4 * tx;
  float4 y[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = ty + 16 * q;
    const float *p = p0 + row * BM;
    float4 t = *reinterpret_cast<const float4 *>(p);
    for (int k = 1; k < a.S; ++k) {
      const float4 u = *reinterpret_cast<const float4 *>(p + (int64_t)k * (BM * BM));
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    y[q] = make_float4(t.x * s, t.y * s, t.z * s, t.w * s);
    const int64_t r = R0 + row, c = C0 + 4 * tx;  // m % 16 == 0: c < m covers c + 3
    if (r < a.m && c < a.m) {
      float4 o = y[q];
      if (a.cin) {
        const float4 x = *reinterpret_cast<const float4 *>(a.cin + r * a.ldcin + c);
        o.x += a.beta * x.x;
        o.y += a.beta * x.y;
        o.z += a.beta * x.z;
        o.w += a.beta * x.w;
      }
      *reinterpret_cast<float4 *>(a.c + r * a.ldc + c) = o;
    }
  }
  if (I == J) return;  // a diagonal tile holds both orders itself (block-uniform)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = ty + 16 * q;
    tr[row][4 * tx] = y[q].x;
    tr[row][4 * tx + 1] = y[q].y;
    tr[row][4 * tx + 2] = y[q].z;
    tr[row][4 * tx + 3] = y[q].w;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int mr = ty + 16 * q;  // the mirror's row: column mr of the sub-block
    const int64_t r = C0 + mr, c = R0 + 4 * tx;
    if (r < a.m && c < a.m) {
      float4 o = make_float4(tr[4 * tx][mr], tr[4 * tx + 1][mr], tr[4 * tx + 2][mr], tr[4 * tx + 3][mr]);
      if (a.cin) {
        const float4 x = *reinterpret_cast<const float4 *>(a.cin + r * a.ldcin + c);
        o.x += a.beta * x.x;
        o.y += a.beta * x.y;
        o.z += a.beta * x.z;
        o.w += a.beta * x.w;
      }
      *reinterpret_cast<float4 *>(a.c + r * a.ldc + c) = o;
    }
  }
}

// Tiles per side, tile pairs, splits and K steps per split of a symmetric
// split-K product, or splits < 2 where it does not apply.
struct SymPlan {
  int T, P, S, steps;
};

SymPlan sym_plan(int64_t m, int64_t K) {
  SymPlan p{0, 0, 0, 0};
  if (m <= 0 || K <= 0 || K % BK || m % 16 || !w8_applies(m, m, K)) return p;
  const int64_t T = (m + BM - 1) / BM, P = T * (T + 1) / 2, ks = K / BK;
  if (P > 128) return p;
  int64_t S = std::min<int64_t>(256 / P, ks);
  if (S < 2) return p;
  const int64_t steps = (ks + S - 1) / S;
  S = (ks + steps - 1) / steps;  // no empty split
  if (S < 2) return p;
  p = SymPlan{(int)T, (int)P, (int)S, (int)steps};
  return p;
}

}  // namespace

size_t gemm_symmetric_partial_bytes(int64_t m, int64_t K) {
  const SymPlan p = sym_plan(m, K);
  return p.S < 2 ? 0 : (size_t)p.P * p.S * BM * BM * sizeof(float);
}

nvfp4_status launch_gemm_symmetric(const GemmProblem &p, float *part, size_t part_bytes, hipStream_t s) {
  auto a16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (p.batch != 1 || p.M != p.N || p.a_codes != p.b_codes || p.a_scales != p.b_scales || p.a_st != p.b_st ||
      p.c_bf16 || p.c_transposed || p.lr_t || p.ldc % 4 || !a16(p.c) ||
      (p.cin && (p.ldcin % 4 || !a16(p.cin))) || p.tile_m || p.tile_n)
    return NVFP4_EUNSUPPORTED;
  const SymPlan sp = sym_plan(p.M, p.K);
  if (sp.S < 2) return NVFP4_EUNSUPPORTED;
  if (!part || part_bytes < (size_t)sp.P * sp.S * BM * BM * sizeof(float) || !a16(part)) return NVFP4_EWORKSPACE;
  GemmArgs g{};
  g.a_codes = p.a_codes;
  g.a_scales = p.a_scales;
  g.a_st = p.a_st;
  g.b_codes = p.b_codes;
  g.b_scales = p.b_scales;
  g.b_st = p.b_st;
  g.M = p.M;
  g.N = p.N;
  g.K = p.K;
  g.alpha = p.alpha;
  g.sym_t = sp.T;
  g.sym_splits = sp.S;
  g.sym_steps = sp.steps;
  g.sym_part = part;
  hipLaunchKernelGGL((gemm_nvfp4_kernel<4, true, false, true, true>), dim3((unsigned)(sp.P * sp.S)), dim3(kThreads),
                     0, s, g);
  SymArgs r{part, sp.T, sp.S, p.M, p.a_st, p.b_st, p.alpha, p.cin, p.ldcin, p.beta, static_cast<float *>(p.c), p.ldc};
  hipLaunchKernelGGL(sym_reduce_kernel, dim3((unsigned)(sp.P * 16)), dim3(256), 0, s, r);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

double gemm_tile_cost(int64_t M, int64_t N, int64_t K, int64_t batch) {
  return pick_tiles(M, N, batch, w8_applies(M, N, K), 0, 0, false).cost;
}

nvfp4_status launch_gemm(const GemmProblem &p, hipStream_t s) {
  if (p.batch == 0 || p.M == 0 || p.N == 0) return NVFP4_OK;
  if (p.batch > 65535) return NVFP4_EUNSUPPORTED;
  GemmArgs g{};
  g.a_codes = p.a_codes;
  g.a_scales = p.a_scales;
  g.a_st = p.a_st;
  g.b_codes = p.b_codes;
  g.b_scales = p.b_scales;
  g.b_st = p.b_st;
  g.M = p.M;
  g.N = p.N;
  g.K = p.K;
  g.c = p.c;
  g.ldc = p.ldc;
  g.bstride_c = p.bstride_c;
  g.alpha = p.alpha;
  g.cin = p.cin;
  g.ldcin = p.ldcin;
  g.bstride_cin = p.bstride_cin;
  g.beta = p.beta;
  g.lr_t = p.lr_t;
  g.lr_l2 = p.lr_l2;
  g.lr_r = p.lr_r;
  g.lr_beta = p.lr_beta;
  g.ct = p.c_transposed;
  auto a16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool c_vec = !p.c_bf16 && p.ldc % 4 == 0 && p.bstride_c % 4 == 0 && a16(p.c);
  const bool cin_vec = !p.cin || (p.ldcin % 4 == 0 && p.bstride_cin % 4 == 0 && a16(p.cin));
  if (g.ct) {
    if (p.c_bf16 || p.lr_t) return NVFP4_EUNSUPPORTED;
    if (!c_vec || !cin_vec) return NVFP4_EALIGN;
  }
  g.staged = c_vec && cin_vec && (g.ct || p.cin);
  const bool fast = p.K % BK == 0;
  // operands small enough for 32-bit load offsets (the 8-wavefront kernels, the 4-wavefront offset variant)
  const bool small = p.M * (p.K / 2) < ((int64_t)1 << 31) && p.N * (p.K / 2) < ((int64_t)1 << 31) &&
                     p.M < (1 << 24) && p.N < (1 << 24) && p.K / 2 < (1 << 24);
  const TilePick tp = pick_tiles(p.M, p.N, p.batch, w8_applies(p.M, p.N, p.K), p.tile_m, p.tile_n, p.lr_t != nullptr);
  if (tp.kind < 0) return NVFP4_EUNSUPPORTED;
  const int64_t tm = (p.M + tp.bm - 1) / tp.bm, tn = (p.N + tp.bn - 1) / tp.bn;
  if (tm * tn > 0x7FFFFFFF) return NVFP4_EUNSUPPORTED;
  g.tiles_m = (int)tm;
  g.tiles_n = (int)tn;
  hipError_t e;
  if (tp.kind == 10) e = launch_w8<4, 2>(g, p.batch, p.c_bf16, s);
  else if (tp.kind == 11) e = launch_w8<2, 4>(g, p.batch, p.c_bf16, s);
  else if (tp.kind == 4) e = launch_tiles<4>(g, p.batch, fast, p.c_bf16, small, s);
  else if (tp.kind == 3) e = launch_tiles<3>(g, p.batch, fast, p.c_bf16, small, s);
  else e = launch_tiles<2>(g, p.batch, fast, p.c_bf16, small, s);
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace nvfp4
