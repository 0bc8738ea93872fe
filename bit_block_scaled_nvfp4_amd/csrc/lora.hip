// lora.hip -- the BF16 down-projection of a LoRA-style layer ("Full-Stack
// FP4 ...", section 2.1: W = W_res + beta L2 L1, the compact subspace L2 L1
// kept in BF16 while W_res runs in NVFP4): T = BF16_RNE(X L1^T) with FP32
// accumulation on the BF16 MFMA.  The up-projection beta T L2^T is folded
// into the NVFP4 GEMM's epilogue (gemm.hip).
//
// Workgroup: 32 rows of X, eight (four for r > 64) wavefronts splitting K;
// each wave keeps ceil(r/32) accumulator fragments (all of T's columns, so X
// is read once), the waves' partial sums meet in LDS and are added in wave
// order (deterministic), rounded to BF16 and stored.  Operands come
// straight from global memory: lane l loads 8 BF16 of row l % 32 at 8 (l/32)
// within each 16-wide step, the same layout for X and L1.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_codec.hpp"
#include "internal.hpp"

namespace nvfp4 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kDownUnroll = 4;
// Eight wavefronts where the accumulators leave room for two per SIMD.
constexpr int down_waves(int f) { return f <= 2 ? 8 : 4; }

struct DownArgs {
  const uint16_t *x;  // [M][K], row stride ldx
  int64_t M, K, ldx;
  const uint16_t *l1;  // [r][K] contiguous
  int64_t r;
  uint16_t *t;  // [M][r] contiguous
};

template <int kF>  // accumulator fragments: ceil(r / 32)
__global__ __launch_bounds__(64 * down_waves(kF)) void lora_down_kernel(DownArgs a) {
  constexpr int kDownWaves = down_waves(kF);
  __shared__ floatx16 part[kDownWaves - 1][kF][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, k8 = 8 * (lane >> 5);
  const int64_t row = min((int64_t)blockIdx.x * 32 + r32, a.M - 1);
  const int64_t steps = a.K / 16;
  const int64_t s0 = steps * wave / kDownWaves, s1 = steps * (wave + 1) / kDownWaves;
  floatx16 acc[kF];
#pragma unroll
  for (int f = 0; f < kF; ++f) acc[f] = floatx16{};
  const uint16_t *xr = a.x + row * a.ldx + k8;
  // Rows of L1 past r (when r % 32 == 16) are read clamped and zeroed.
  const uint16_t *lr[kF];
  bool lok[kF];
#pragma unroll
  for (int f = 0; f < kF; ++f) {
    const int64_t l = 32 * f + r32;
    lok[f] = l < a.r;
    lr[f] = a.l1 + min(l, a.r - 1) * a.K + k8;
  }
  int64_t s = s0;
  for (; s + kDownUnroll <= s1; s += kDownUnroll) {
    bf16x8_t xa[kDownUnroll], lb[kDownUnroll][kF];
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u) {
      xa[u] = *reinterpret_cast<const bf16x8_t *>(xr + 16 * (s + u));
#pragma unroll
      for (int f = 0; f < kF; ++f) lb[u][f] = *reinterpret_cast<const bf16x8_t *>(lr[f] + 16 * (s + u));
    }
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u)
#pragma unroll
      for (int f = 0; f < kF; ++f) {
        const bf16x8_t b = lok[f] ? lb[u][f] : bf16x8_t{};
        acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[u], b, acc[f], 0, 0, 0);
      }
  }
  for (; s < s1; ++s) {
    const bf16x8_t xa = *reinterpret_cast<const bf16x8_t *>(xr + 16 * s);
#pragma unroll
    for (int f = 0; f < kF; ++f) {
      const bf16x8_t lb = *reinterpret_cast<const bf16x8_t *>(lr[f] + 16 * s);
      acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, lok[f] ? lb : bf16x8_t{}, acc[f], 0, 0, 0);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int f = 0; f < kF; ++f) part[wave - 1][f][lane] = acc[f];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kDownWaves - 1; ++w)
#pragma unroll
    for (int f = 0; f < kF; ++f) acc[f] += part[w][f][lane];
  // Accumulator v of lane l: row 8 (v/4) + 4 (l/32) + v%4, column l % 32.
  const int h = lane >> 5;
#pragma unroll
  for (int f = 0; f < kF; ++f) {
    const int64_t col = 32 * f + r32;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const int64_t r0 = (int64_t)blockIdx.x * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      const uint32_t b2 = pack_bf16x2_rne(acc[f][v], acc[f][v + 1]);
      if (col < a.r) {
        if (r0 < a.M) a.t[r0 * a.r + col] = (uint16_t)b2;
        if (r0 + 1 < a.M) a.t[(r0 + 1) * a.r + col] = (uint16_t)(b2 >> 16);
      }
    }
  }
}

}  // namespace

nvfp4_status launch_lora_down(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint16_t *l1, int64_t r,
                              uint16_t *t, hipStream_t s) {
  if (M <= 0 || r <= 0) return NVFP4_OK;
  if (K % 16 || r % 16 || r > 128 || (M + 31) / 32 > 0x7FFFFFFF) return NVFP4_EUNSUPPORTED;
  DownArgs a{x, M, K, ldx, l1, r, t};
  const dim3 grid((unsigned)((M + 31) / 32));
  switch ((r + 31) / 32) {
    case 1: hipLaunchKernelGGL(lora_down_kernel<1>, grid, dim3(64 * down_waves(1)), 0, s, a); break;
    case 2: hipLaunchKernelGGL(lora_down_kernel<2>, grid, dim3(64 * down_waves(2)), 0, s, a); break;
    case 3: hipLaunchKernelGGL(lora_down_kernel<3>, grid, dim3(64 * down_waves(3)), 0, s, a); break;
    default: hipLaunchKernelGGL(lora_down_kernel<4>, grid, dim3(64 * down_waves(4)), 0, s, a); break;
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace nvfp4
