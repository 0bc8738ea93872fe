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
// The decode is the VALU cost: the FP4 -> FP16 converter issues at about half
// the rate of a plain VALU instruction, so decoding one fragment's sub-step
// (8 elements per lane) costs about as much issue time as 1.5 MFMAs, and with
// one wavefront per SIMD it only overlaps the matrix pipe when it sits
// between MFMAs of other operands.  Three main loops:
//  * K % 128 == 0, tiles 256 x 192 / 256 x 128: software pipelined.  The next
//    sub-step is decoded while the current one's MFMAs run (grouped one MFMA
//    to a few VALU instructions), codes are read from LDS half a step ahead,
//    and global_load_lds fills the stage of the step after next, so global
//    latency has a whole step and LDS latency half a step to hide.
//  * K % 128 == 0, tiles 256 x 256: the accumulators fill the AGPR file, so
//    a step reads its codes from LDS, issues the next step's global_load_lds
//    (into the idle stage, no VGPRs), then decodes and multiplies.
//  * Other K: register-staged loads with the K tail read as zero codes and
//    scales (zero products).
// The launcher picks the tile width so that the tile count fills the 256
// CUs in whole rounds.
//
// Workgroups are mapped to tiles so that each XCD (blockIdx mod 8 under the
// round-robin dispatch) works on a contiguous range of tiles, in groups of
// kGroupM tile rows, to keep A and B panels in that XCD's L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.hpp"

#ifndef NVFP4_GEMM_INTERLEAVE
#define NVFP4_GEMM_INTERLEAVE 5
#endif
#ifndef NVFP4_GEMM_SWIZZLE
#define NVFP4_GEMM_SWIZZLE 2
#endif

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kRowBytes = BK / 2;  // 64 code bytes per row per K step
constexpr int kFragM = 4;          // 32-row A fragments per wavefront
constexpr int kGroupM = 8;         // tile rows per L2 group
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// LDS placement of the 16-byte code chunk `part` (0..3) of tile row `row`.
// Fragment reads take the same part from 32 consecutive rows; XOR-ing the
// part with row bits spreads those reads over all LDS banks.
__device__ __forceinline__ int chunk_slot(int row, int part) {
#if NVFP4_GEMM_SWIZZLE == 1
  return row * 4 + (part ^ ((row >> 1) & 3));
#elif NVFP4_GEMM_SWIZZLE == 2
  return row * 4 + (part ^ ((row >> 2) & 3));
#else
  return row * 4 + part;
#endif
}

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
};

// LDS stage: codes [rows][64 B] and scales [rows][8 B] per operand.
template <int kBN>
struct alignas(16) Stage {
  uint8_t a[BM * kRowBytes];
  uint8_t b[kBN * kRowBytes];
  uint2 as[BM];
  uint2 bs[kBN];
};

// Two E4M3 scale bytes (bits 0..6 and 8..14 of w) -> two FP16 scales in one
// dword.  An E4M3 code c shifted left by 7 and read as FP16 is c's value
// times 2^-8 (the exponent fields line up; subnormal codes become FP16
// subnormals), so one packed multiply by 256 gives the exact values.
__device__ __forceinline__ half2_t scale_pair2(uint32_t w) {
  const uint32_t spread = __builtin_amdgcn_perm(0u, w, 0x0C010C00u);  // [s0, 0, s1, 0]
  const half2_t k256 = {(_Float16)256.0f, (_Float16)256.0f};
  return __builtin_bit_cast(half2_t, spread << 7) * k256;
}

// Eight E2M1 codes (element 2j in the low nibble of byte j) times one FP16
// block scale -> eight FP16 values in element order.
__device__ __forceinline__ half8_t decode8(uint32_t codes, _Float16 s) {
  const half2_t s2 = {s, s};
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Direct global -> LDS loads of one operand's K step (K % 128 == 0): each
// wavefront's global_load_lds fills 64 consecutive lane slots, which keeps
// the row-major [rows][64 B] code and [rows][8 B] scale layout.  Rows past
// the end are clamped; their products only reach output rows never stored.
template <int kRows>
__device__ __forceinline__ void lds_load_operand(const uint8_t *codes_g, const uint8_t *scales_g,
                                                 int64_t rows, int64_t K, int64_t r0, int64_t k0,
                                                 uint8_t *lds_codes, uint2 *lds_scales) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t kblocks = K / 16;
  constexpr int kCodeLoads = kRows * 4 / kThreads;  // 16-byte chunks per lane
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
  constexpr int kScaleLoads = (kRows * 2 + kThreads - 1) / kThreads;  // dwords per lane
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
    sc.a[f][0] = scale_pair2(w);
    sc.a[f][1] = scale_pair2(w >> 16);
  }
#pragma unroll
  for (int f = 0; f < kFragN; ++f) {
    const int row = c.wn * (32 * kFragN) + f * 32 + c.r32;
    const uint32_t w = c.h ? st.bs[row].y : st.bs[row].x;
    sc.b[f][0] = scale_pair2(w);
    sc.b[f][1] = scale_pair2(w >> 16);
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
  for (int f = 0; f < kFragM; ++f) av[f] = decode8(word_at<kS & 3>(r.a[f]), sc.a[f][kS >> 2][(kS >> 1) & 1]);
#pragma unroll
  for (int f = 0; f < kFragN; ++f) bv[f] = decode8(word_at<kS & 3>(r.b[f]), sc.b[f][kS >> 2][(kS >> 1) & 1]);
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
#if NVFP4_GEMM_INTERLEAVE
  // One wavefront per SIMD issues in order, so VALU work only overlaps an
  // MFMA if it sits between MFMAs: ask for kFragM * kFragN groups of one
  // MFMA followed by a few VALU instructions.
#pragma unroll
  for (int i = 0; i < kFragM * kFragN; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_GEMM_INTERLEAVE, 0);
  }
#endif
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
template <int kFragN, int kBN>
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
    lds_load_operand<BM>(t.ac, t.as, t.M, t.K, t.m0, k0, cur.a, cur.as);
    lds_load_operand<kBN>(t.bc, t.bs, t.N, t.K, t.n0, k0, cur.b, cur.bs);
  }
  mfma_and_decode<5>(r1, sc_cur, av, bv, acc);
  mfma_and_decode<6>(r1, sc_cur, av, bv, acc);
  mfma_and_decode<7>(r1, sc_cur, av, bv, acc);
  mfma_and_decode<0>(r0, sc_nxt, av, bv, acc);
}

template <int kFragN, bool kFast, bool kBF16Out>
__global__ __launch_bounds__(kThreads) void gemm_nvfp4_kernel(GemmArgs g) {
  constexpr int kBN = 64 * kFragN;
  // Two stages as separate objects: the compiler can then tell a read of one
  // from a global->LDS load in flight into the other and does not wait for it.
  __shared__ Stage<kBN> st0, st1;

  // XCD-aware tile order: consecutive workgroups go to different XCDs, so
  // give XCD x the x-th contiguous slice of the grouped tile order.
  const int ntiles = g.tiles_m * g.tiles_n;
  const int bid = blockIdx.x;
  const int per_xcd = ntiles / 8;
  const int t = (ntiles % 8 == 0) ? (bid % 8) * per_xcd + bid / 8 : bid;
  const int group = t / (kGroupM * g.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(g.tiles_m - first_m, kGroupM);
  const int in_group = t - group * kGroupM * g.tiles_n;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;

  const int64_t batch = blockIdx.y;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * kBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  const uint8_t *ac = g.a_codes + batch * g.M * (g.K / 2);
  const uint8_t *as = g.a_scales + batch * g.M * (g.K / 16);
  const uint8_t *bc = g.b_codes + batch * g.N * (g.K / 2);
  const uint8_t *bs = g.b_scales + batch * g.N * (g.K / 16);

  floatx16 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int ksteps = (int)((g.K + BK - 1) / BK);
  if constexpr (kFast && kFragN <= 3) {
    const TileSrc src{ac, as, bc, bs, g.M, g.N, g.K, m0, n0};
    const LaneCoord c{wm, wn, h, r32};
    if (ksteps > 0) {
      lds_load_operand<BM>(ac, as, g.M, g.K, m0, 0, st0.a, st0.as);
      lds_load_operand<kBN>(bc, bs, g.N, g.K, n0, 0, st0.b, st0.bs);
      if (ksteps > 1) {
        lds_load_operand<BM>(ac, as, g.M, g.K, m0, BK, st1.a, st1.as);
        lds_load_operand<kBN>(bc, bs, g.N, g.K, n0, BK, st1.b, st1.bs);
      }
    }
    __syncthreads();
    HalfCodes<kFragN> r0, r1;
    StepScales<kFragN> sc0, sc1;  // scales of even / odd steps
    half8_t av[kFragM], bv[kFragN];
    read_codes<kFragN>(st0, 0, c, r0);
    read_scales<kFragN>(st0, c, sc0);
    decode_substep<0, kFragN>(r0, sc0, av, bv);
    for (int kt = 0; kt < ksteps; kt += 2) {
      pipelined_kstep<kFragN>(st0, st1, src, kt, ksteps, c, r0, r1, sc0, sc1, av, bv, acc);
      if (kt + 1 < ksteps) pipelined_kstep<kFragN>(st1, st0, src, kt + 1, ksteps, c, r0, r1, sc1, sc0, av, bv, acc);
    }
  } else if constexpr (kFast) {
    // 256 x 256 tiles: the accumulators take all 256 AGPRs, which leaves no
    // room for the pipelined loop's second code and operand buffers.  A K
    // step reads its codes from LDS, issues the global->LDS loads of the
    // next step, then decodes and multiplies.
    if (ksteps > 0) {
      lds_load_operand<BM>(ac, as, g.M, g.K, m0, 0, st0.a, st0.as);
      lds_load_operand<kBN>(bc, bs, g.N, g.K, n0, 0, st0.b, st0.bs);
    }
    __syncthreads();
    for (int kt = 0; kt < ksteps; ++kt) {
      const Stage<kBN> &cur = (kt & 1) ? st1 : st0;
      Stage<kBN> &nxt = (kt & 1) ? st0 : st1;
      uint4 ca[kFragM][2], cb[kFragN][2];
      half2_t sa[kFragM][2], sb[kFragN][2];
#pragma unroll
      for (int f = 0; f < kFragM; ++f) {
        const int r = wm * 128 + f * 32 + r32;
        ca[f][0] = *reinterpret_cast<const uint4 *>(cur.a + 16 * chunk_slot(r, 2 * h));
        ca[f][1] = *reinterpret_cast<const uint4 *>(cur.a + 16 * chunk_slot(r, 2 * h + 1));
        const uint32_t w = h ? cur.as[r].y : cur.as[r].x;
        sa[f][0] = scale_pair2(w);
        sa[f][1] = scale_pair2(w >> 16);
      }
#pragma unroll
      for (int f = 0; f < kFragN; ++f) {
        const int r = wn * (32 * kFragN) + f * 32 + r32;
        cb[f][0] = *reinterpret_cast<const uint4 *>(cur.b + 16 * chunk_slot(r, 2 * h));
        cb[f][1] = *reinterpret_cast<const uint4 *>(cur.b + 16 * chunk_slot(r, 2 * h + 1));
        const uint32_t w = h ? cur.bs[r].y : cur.bs[r].x;
        sb[f][0] = scale_pair2(w);
        sb[f][1] = scale_pair2(w >> 16);
      }
      // Issued after this step's LDS reads, so no read waits on them.
      if (kt + 1 < ksteps) {
        lds_load_operand<BM>(ac, as, g.M, g.K, m0, (int64_t)(kt + 1) * BK, nxt.a, nxt.as);
        lds_load_operand<kBN>(bc, bs, g.N, g.K, n0, (int64_t)(kt + 1) * BK, nxt.b, nxt.bs);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        half8_t av[kFragM], bv[kFragN];
#pragma unroll
        for (int f = 0; f < kFragM; ++f) av[f] = decode8(word_of(ca[f][s >> 2], s & 3), sa[f][s >> 2][(s >> 1) & 1]);
#pragma unroll
        for (int f = 0; f < kFragN; ++f) bv[f] = decode8(word_of(cb[f][s >> 2], s & 3), sb[f][s >> 2][(s >> 1) & 1]);
        mfma_substep<kFragN>(acc, av, bv);
      }
      // The next stage must have landed before the barrier.  The scheduling
      // fences keep the wait below this step's math (hoisted, it would wait
      // for the loads just issued) and the MFMAs above the barrier.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
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
        sa[f][0] = scale_pair2(w);
        sa[f][1] = scale_pair2(w >> 16);
      }
#pragma unroll
      for (int f = 0; f < kFragN; ++f) {
        const int r = wn * (32 * kFragN) + f * 32 + r32;
        cb[f][0] = *reinterpret_cast<const uint4 *>(cur.b + 16 * chunk_slot(r, 2 * h));
        cb[f][1] = *reinterpret_cast<const uint4 *>(cur.b + 16 * chunk_slot(r, 2 * h + 1));
        const uint32_t w = h ? cur.bs[r].y : cur.bs[r].x;
        sb[f][0] = scale_pair2(w);
        sb[f][1] = scale_pair2(w >> 16);
      }
      if (more) {
        la.load(ac, as, g.M, g.K, m0, (int64_t)(kt + 1) * BK);
        lb.load(bc, bs, g.N, g.K, n0, (int64_t)(kt + 1) * BK);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        half8_t av[kFragM], bv[kFragN];
#pragma unroll
        for (int f = 0; f < kFragM; ++f) av[f] = decode8(word_of(ca[f][s >> 2], s & 3), sa[f][s >> 2][(s >> 1) & 1]);
#pragma unroll
        for (int f = 0; f < kFragN; ++f) bv[f] = decode8(word_of(cb[f][s >> 2], s & 3), sb[f][s >> 2][(s >> 1) & 1]);
        mfma_substep<kFragN>(acc, av, bv);
      }
      if (more) {
        la.store(nxt.a, nxt.as);
        lb.store(nxt.b, nxt.bs);
      }
      __syncthreads();
    }
  }

  // Epilogue: multiply by fl(fl(sA * sB) * alpha) and store.  Accumulator v
  // of lane l in a 32x32 tile holds row 8*(v/4) + 4*(l/32) + v%4, column l%32.
  using OutT = typename std::conditional<kBF16Out, uint16_t, float>::type;
  const float sc = (*g.a_st * *g.b_st) * g.alpha;
  OutT *cb_ptr = static_cast<OutT *>(g.c) + batch * g.bstride_c;
  const int64_t row0 = m0 + wm * 128 + 4 * h;
  const int64_t col0 = n0 + wn * (32 * kFragN) + r32;
  int64_t roff[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) roff[v] = (int64_t)(8 * (v >> 2) + (v & 3)) * g.ldc;
  const bool full = m0 + BM <= g.M && n0 + kBN <= g.N;
#pragma unroll
  for (int i = 0; i < kFragM; ++i) {
    OutT *prow = cb_ptr + (row0 + 32 * i) * g.ldc + col0;
#pragma unroll
    for (int j = 0; j < kFragN; ++j) {
      const bool col_ok = full || col0 + 32 * j < g.N;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int64_t r = row0 + 32 * i + 8 * (v >> 2) + (v & 3);
        const bool ok0 = col_ok && (full || r < g.M), ok1 = col_ok && (full || r + 1 < g.M);
        if constexpr (kBF16Out) {
          // v_cvt_pk_bf16_f32: two FP32 -> BF16, round to nearest even
          const float2_t y2 = {acc[i][j][v] * sc, acc[i][j][v + 1] * sc};
          const uint32_t b2 = __builtin_bit_cast(uint32_t, __builtin_convertvector(y2, bf16x2_t));
          if (ok0) prow[roff[v] + 32 * j] = (uint16_t)b2;
          if (ok1) prow[roff[v + 1] + 32 * j] = (uint16_t)(b2 >> 16);
        } else {
          if (ok0) prow[roff[v] + 32 * j] = acc[i][j][v] * sc;
          if (ok1) prow[roff[v + 1] + 32 * j] = acc[i][j][v + 1] * sc;
        }
      }
    }
  }
}

template <int kFragN>
hipError_t launch_tiles(const GemmArgs &g, int64_t batch, bool fast, bool bf16, hipStream_t s) {
  const dim3 grid((unsigned)(g.tiles_m * g.tiles_n), (unsigned)batch);
  if (fast && bf16)
    hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, true, true>), grid, dim3(kThreads), 0, s, g);
  else if (fast)
    hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, true, false>), grid, dim3(kThreads), 0, s, g);
  else if (bf16)
    hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, false, true>), grid, dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_nvfp4_kernel<kFragN, false, false>), grid, dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

// N-tile width (64 * kFragN): among 256, 192 and 128, the one with the least
// estimated time, counting a partly filled last round of workgroups as a full
// round (one workgroup per CU, 256 CUs) and costing narrower tiles by their
// extra decode work per MFMA (measured on fprop/MLP-sized problems).
int pick_frag_n(int64_t M, int64_t N, int64_t batch) {
  const int64_t tm = (M + BM - 1) / BM;
  double best = 1e300;
  int pick = 4;
  const int cands[3] = {4, 3, 2};
  const double cost_per_col[3] = {1.0, 1.02, 1.12};
  for (int c = 0; c < 3; ++c) {
    const int fn = cands[c];
    const int64_t tn = (N + 64 * fn - 1) / (64 * fn);
    const int64_t tiles = tm * tn * batch;
    const int64_t rounds = (tiles + 255) / 256;
    const double t = (double)rounds * (double)(64 * fn) * cost_per_col[c];
    if (t < best - 1e-9) {
      best = t;
      pick = fn;
    }
  }
#ifdef NVFP4_GEMM_FORCE_FRAG_N
  pick = NVFP4_GEMM_FORCE_FRAG_N;
#endif
  return pick;
}

}  // namespace

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
  const bool fast = p.K % BK == 0;
  const int fn = pick_frag_n(p.M, p.N, p.batch);
  const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + 64 * fn - 1) / (64 * fn);
  if (tm * tn > 0x7FFFFFFF) return NVFP4_EUNSUPPORTED;
  g.tiles_m = (int)tm;
  g.tiles_n = (int)tn;
  hipError_t e;
  if (fn == 4) e = launch_tiles<4>(g, p.batch, fast, p.c_bf16, s);
  else if (fn == 3) e = launch_tiles<3>(g, p.batch, fast, p.c_bf16, s);
  else e = launch_tiles<2>(g, p.batch, fast, p.c_bf16, s);
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace nvfp4
