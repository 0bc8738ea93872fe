// hw_probe.hip -- test infrastructure, not part of the library.  Runs the
// library's own device codec functions (bit_block_scaled_nvfp4_amd/csrc/
// device_codec.hpp: the E2M1 round-to-nearest-even, stochastic-rounding and
// BF16 hardware converters as the kernels use them, and the E4M3 block-scale
// encode) over inputs the tests choose, so that
// tests/test_hw_converters.py can compare them with the CPU oracle over
// every FP32 bit pattern.  Every kernel checks its index against the count
// it is given; the host wrappers launch one thread per output unit.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../bit_block_scaled_nvfp4_amd/csrc/device_codec.hpp"

namespace {

using namespace nvfp4;
constexpr int kBlock = 256;

unsigned blocks_for(uint64_t n) { return (unsigned)((n + kBlock - 1) / kBlock); }

// Codes of FP32 patterns first + 8t .. first + 8t + 7 (mod 2^32), packed
// as the quantize kernels pack them: element j in nibble j.
__global__ void k_e2m1_rne8(uint32_t first, uint64_t ngroups, uint32_t *out) {
  const uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= ngroups) return;
  float q[8];
  for (int j = 0; j < 8; ++j) q[j] = __uint_as_float(first + (uint32_t)(8 * t) + (uint32_t)j);
  out[t] = e2m1_rne8(q);
}

// E4M3 block-scale code of FP32 pattern first + t.
__global__ void k_e4m3(uint32_t first, uint64_t n, uint8_t *out) {
  const uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= n) return;
  out[t] = (uint8_t)e4m3_encode(__uint_as_float(first + (uint32_t)t));
}

// Stochastic rounding of q[i] under word u through e2m1_sr8 with all eight
// elements equal to q[i] and every 16-bit half of the words equal to u:
// out[i * 65536 + u] = byte 0 of the result (the low lane's code | the high
// lane's code << 4); *bad counts results whose four bytes differ.
__global__ void k_e2m1_sr(const float *q, uint64_t nq, uint8_t *out, unsigned long long *bad) {
  const uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= nq * 65536) return;
  const float v = q[t >> 16];
  const uint32_t u = (uint32_t)(t & 0xFFFFu), w = u | (u << 16);
  const float q8[8] = {v, v, v, v, v, v, v, v};
  const uint32_t c = e2m1_sr8(q8, w, w, w, w);
  if ((c & 0xFFu) * 0x01010101u != c) atomicAdd(bad, 1ull);
  out[t] = (uint8_t)(c & 0xFFu);
}

// For every FP32 pattern first + t: the codes at the two words around its
// rounding threshold U = ceil(floor(f * 2^22) / 64) (the words below U round
// up), U - 1 and U (clamped to 0..65535), each through e2m1_sr8 with all
// eight elements equal to the value: out[t] = byte 0 as above for U - 1 in
// the low byte, for U in the high byte; *bad counts results whose four bytes
// differ.
__global__ void k_sr_threshold(uint32_t first, uint64_t n, uint16_t *out, unsigned long long *bad) {
  const uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= n) return;
  const float v = __uint_as_float(first + (uint32_t)t);
  const float a = fminf(fabsf(v), 6.0f);
  const uint32_t eb = __float_as_uint(a) >> 23;
  const uint32_t e = (eb > 127u ? eb : 127u) - 127u;
  const float tt = __builtin_ldexpf(a, 1 - (int)e);
  const uint32_t F = (uint32_t)(__builtin_amdgcn_fractf(tt) * 4194304.0f);
  const uint32_t U = (F + 63u) / 64u;
  const uint32_t us[2] = {U == 0u ? 0u : U - 1u, U > 65535u ? 65535u : U};
  const float q8[8] = {v, v, v, v, v, v, v, v};
  uint32_t res = 0;
  for (int k = 0; k < 2; ++k) {
    const uint32_t w = us[k] | (us[k] << 16);
    const uint32_t c = e2m1_sr8(q8, w, w, w, w);
    if ((c & 0xFFu) * 0x01010101u != c) atomicAdd(bad, 1ull);
    res |= (c & 0xFFu) << (8 * k);
  }
  out[t] = (uint16_t)res;
}

// BF16 of FP32 patterns first + 2t (low half) and first + 2t + 1 (high half).
__global__ void k_bf16(uint32_t first, uint64_t npairs, uint32_t *out) {
  const uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= npairs) return;
  const uint32_t p = first + (uint32_t)(2 * t);
  out[t] = pack_bf16x2_rne(__uint_as_float(p), __uint_as_float(p + 1u));
}

int status() { return hipGetLastError() == hipSuccess ? 0 : 1; }

}  // namespace

#define PROBE_EXPORT extern "C" __attribute__((visibility("default")))

// n % 8 == 0; out: n / 2 bytes.
PROBE_EXPORT int hwprobe_e2m1_rne8(uint32_t first, int64_t n, void *out, void *stream) {
  if (n <= 0 || n % 8) return 2;
  hipLaunchKernelGGL(k_e2m1_rne8, dim3(blocks_for(n / 8)), dim3(kBlock), 0, (hipStream_t)stream, first,
                     (uint64_t)(n / 8), (uint32_t *)out);
  return status();
}

// out: n bytes.
PROBE_EXPORT int hwprobe_e4m3(uint32_t first, int64_t n, void *out, void *stream) {
  if (n <= 0) return 2;
  hipLaunchKernelGGL(k_e4m3, dim3(blocks_for(n)), dim3(kBlock), 0, (hipStream_t)stream, first, (uint64_t)n,
                     (uint8_t *)out);
  return status();
}

// q: nq device floats; out: nq * 65536 bytes; bad: one device counter.
PROBE_EXPORT int hwprobe_e2m1_sr(const void *q, int64_t nq, void *out, void *bad, void *stream) {
  if (nq <= 0) return 2;
  hipLaunchKernelGGL(k_e2m1_sr, dim3(blocks_for((uint64_t)nq * 65536)), dim3(kBlock), 0, (hipStream_t)stream,
                     (const float *)q, (uint64_t)nq, (uint8_t *)out, (unsigned long long *)bad);
  return status();
}

// out: n 16-bit values; bad: one device counter.
PROBE_EXPORT int hwprobe_sr_threshold(uint32_t first, int64_t n, void *out, void *bad, void *stream) {
  if (n <= 0) return 2;
  hipLaunchKernelGGL(k_sr_threshold, dim3(blocks_for(n)), dim3(kBlock), 0, (hipStream_t)stream, first, (uint64_t)n,
                     (uint16_t *)out, (unsigned long long *)bad);
  return status();
}

// n % 2 == 0; out: n BF16 values.
PROBE_EXPORT int hwprobe_bf16(uint32_t first, int64_t n, void *out, void *stream) {
  if (n <= 0 || n % 2) return 2;
  hipLaunchKernelGGL(k_bf16, dim3(blocks_for(n / 2)), dim3(kBlock), 0, (hipStream_t)stream, first,
                     (uint64_t)(n / 2), (uint32_t *)out);
  return status();
}
