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
// to 2^-14).  The kernel therefore decodes codes and scales to FP16 in
// registers and runs v_mfma_f32_32x32x16_f16 with FP32 accumulation; only the
// FP32 accumulation order differs from exact arithmetic.  FP16 is chosen over
// BF16 (same MFMA rate on gfx950) because the hardware FP4 -> FP16 converter
// and a packed FP16 multiply decode two elements per instruction each.
//
// Tiling: 128x128 output tile per workgroup of 4 wavefronts (2 x 2, 64x64
// each = 2 x 2 MFMA tiles of 32x32), K step 128 (8 scale blocks).  Per K step
// the workgroup stages 64 code bytes and 8 scale bytes per row of A and B in
// LDS; each lane then reads 32 contiguous code bytes and one scale dword per
// fragment.  Within a K step, lane half h of a fragment covers K offsets
// [64h, 64h + 64): MFMA step s takes K offsets 64h + 8s .. 64h + 8s + 7 from
// half h, which is one 16-element scale block (4h + s/2) per lane.  A and B
// use the same assignment, so every K index meets its partner exactly once.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kCodeBytes = BK / 2;         // 64 code bytes per row per K step
constexpr int kLdsRow = kCodeBytes + 16;   // padded LDS row

struct GemmArgs {
  const uint8_t *a_codes, *a_scales;
  const float *a_st;
  const uint8_t *b_codes, *b_scales;
  const float *b_st;
  int64_t M, N, K;
  int tiles_n;
  void *c;
  int64_t ldc, bstride_c;
  float alpha;
  bool c_bf16;
};

// E4M3 scale byte s -> FP16 pair (S, S).  s << 7 placed in an FP16 is
// S * 2^-8 for every code (the E4M3 exponent field lands in the FP16 one,
// subnormal codes land in FP16 subnormals); one packed multiply by 256 is
// exact and restores S.
__device__ __forceinline__ half2_t scale_pair(uint32_t s) {
  const uint32_t bits = s * 0x00800080u;
  const half2_t k256 = {(_Float16)256.0f, (_Float16)256.0f};
  return __builtin_bit_cast(half2_t, bits) * k256;
}

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times
// the block scale, as eight FP16 values in element order.
__device__ __forceinline__ half8_t decode8(uint32_t codes, half2_t s2) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Global -> registers for one operand tile (rows r0..r0+127, K step k0).
struct StageRegs {
  uint2 codes[4];
  uint32_t scales;
};

__device__ __forceinline__ void stage_load(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                           int64_t K, int64_t r0, int64_t k0, StageRegs &st) {
  const int tid = threadIdx.x;
  const int64_t kblocks = K / 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx >> 3, chunk = idx & 7;
    const int64_t gr = r0 + row, kb = k0 / 16 + chunk;
    st.codes[i] = (gr < rows && kb < kblocks)
                      ? *reinterpret_cast<const uint2 *>(codes + gr * (K / 2) + kb * 8)
                      : make_uint2(0u, 0u);
  }
  {
    const int row = tid >> 1, half = tid & 1;
    const int64_t gr = r0 + row;
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t kb = k0 / 16 + 4 * half + i;
      const uint32_t byte = (gr < rows && kb < kblocks) ? scales[gr * kblocks + kb] : 0u;
      w |= byte << (8 * i);
    }
    st.scales = w;
  }
}

__device__ __forceinline__ void stage_store(const StageRegs &st, uint8_t *lds_codes, uint32_t *lds_scales) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx >> 3, chunk = idx & 7;
    *reinterpret_cast<uint2 *>(lds_codes + row * kLdsRow + chunk * 8) = st.codes[i];
  }
  lds_scales[tid] = st.scales;  // row = tid / 2, dword = tid % 2
}

__global__ __launch_bounds__(kThreads) void gemm_nvfp4_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t sa_codes[BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t sb_codes[BN * kLdsRow];
  __shared__ uint32_t sa_scales[BM * 2];
  __shared__ uint32_t sb_scales[BN * 2];

  const int tile = blockIdx.x;
  const int64_t batch = blockIdx.y;
  const int64_t m0 = (int64_t)(tile / g.tiles_n) * BM;
  const int64_t n0 = (int64_t)(tile % g.tiles_n) * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  const uint8_t *ac = g.a_codes + batch * g.M * (g.K / 2);
  const uint8_t *as = g.a_scales + batch * g.M * (g.K / 16);
  const uint8_t *bc = g.b_codes + batch * g.N * (g.K / 2);
  const uint8_t *bs = g.b_scales + batch * g.N * (g.K / 16);

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  for (int64_t k0 = 0; k0 < g.K; k0 += BK) {
    StageRegs ra, rb;
    stage_load(ac, as, g.M, g.K, m0, k0, ra);
    stage_load(bc, bs, g.N, g.K, n0, k0, rb);
    __syncthreads();
    stage_store(ra, sa_codes, sa_scales);
    stage_store(rb, sb_codes, sb_scales);
    __syncthreads();

    uint4 fa[2][2], fb[2][2];
    uint32_t sca[2], scb[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int ra_row = wm * 64 + f * 32 + r32;
      const int rb_row = wn * 64 + f * 32 + r32;
      fa[f][0] = *reinterpret_cast<const uint4 *>(sa_codes + ra_row * kLdsRow + 32 * h);
      fa[f][1] = *reinterpret_cast<const uint4 *>(sa_codes + ra_row * kLdsRow + 32 * h + 16);
      fb[f][0] = *reinterpret_cast<const uint4 *>(sb_codes + rb_row * kLdsRow + 32 * h);
      fb[f][1] = *reinterpret_cast<const uint4 *>(sb_codes + rb_row * kLdsRow + 32 * h + 16);
      sca[f] = sa_scales[ra_row * 2 + h];
      scb[f] = sb_scales[rb_row * 2 + h];
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t av[2], bv[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const uint4 qa = fa[f][s >> 2], qb = fb[f][s >> 2];
        const uint32_t ca = (s & 3) == 0 ? qa.x : (s & 3) == 1 ? qa.y : (s & 3) == 2 ? qa.z : qa.w;
        const uint32_t cb = (s & 3) == 0 ? qb.x : (s & 3) == 1 ? qb.y : (s & 3) == 2 ? qb.z : qb.w;
        av[f] = decode8(ca, scale_pair((sca[f] >> (8 * (s >> 1))) & 0xFFu));
        bv[f] = decode8(cb, scale_pair((scb[f] >> (8 * (s >> 1))) & 0xFFu));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue: multiply by fl(fl(sA * sB) * alpha), store with bounds checks.
  // Accumulator v of lane l in a 32x32 tile holds row 8*(v/4) + 4*(l/32) + v%4,
  // column l%32.
  const float sc = (*g.a_st * *g.b_st) * g.alpha;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < g.M && col < g.N) {
          const float y = acc[i][j][v] * sc;
          const int64_t off = batch * g.bstride_c + row * g.ldc + col;
          if (g.c_bf16)
            static_cast<uint16_t *>(g.c)[off] = (uint16_t)bf16_rne(y);
          else
            static_cast<float *>(g.c)[off] = y;
        }
      }
    }
}

}  // namespace

nvfp4_status launch_gemm(const GemmProblem &p, hipStream_t s) {
  if (p.batch == 0 || p.M == 0 || p.N == 0) return NVFP4_OK;
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
  const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
  g.tiles_n = (int)tn;
  g.c = p.c;
  g.c_bf16 = p.c_bf16;
  g.ldc = p.ldc;
  g.bstride_c = p.bstride_c;
  g.alpha = p.alpha;
  if (tm * tn > 0x7FFFFFFF || p.batch > 65535) return NVFP4_EUNSUPPORTED;
  hipLaunchKernelGGL(gemm_nvfp4_kernel, dim3((unsigned)(tm * tn), (unsigned)p.batch), dim3(kThreads), 0, s, g);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace nvfp4
