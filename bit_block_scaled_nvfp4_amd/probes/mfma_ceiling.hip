// mfma_ceiling.hip -- sustained rate of v_mfma_f32_32x32x16_f16 on this GPU.
//
// The GEMM decodes NVFP4 operands to FP16 and contracts them with this
// instruction, so its attainable rate bounds the GEMM.  One 256-thread
// workgroup per CU runs 16 independent accumulator chains per wavefront
// (no memory traffic, no other instructions in the loop).  The rate depends
// on the operand bits through power: the chip lowers its clock as more
// multiplier bits toggle.  Three operand sets are timed:
//   const  -- the same small values in every lane (few toggling bits),
//   random -- uniform random FP16 values,
//   nvfp4  -- E2M1 values times E4M3-like scales (1 + m/8) * 2^e, the values
//             the GEMM actually feeds the instruction.
// Prints one JSON line per set: TFLOP/s from HIP events and the average
// shader clock (clock64 over wall_clock64).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t xorshift(uint32_t &x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

__device__ __forceinline__ float operand(int kind, uint32_t &x) {
  const uint32_t r = xorshift(x);
  if (kind == 0) return 0.5f;
  if (kind == 1) return ((int)(r & 0xFFFF) - 32768) * (1.0f / 4096.0f);
  const float e2m1[8] = {0.f, .5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  const float sign = (r >> 3) & 1 ? -1.f : 1.f;
  return e2m1[r & 7] * sign * (1.f + ((r >> 4) & 7) / 8.f) * __builtin_ldexpf(1.f, (int)((r >> 7) % 9) - 4);
}

__global__ __launch_bounds__(256) void mfma_loop(int kind, int iters, float *sink, unsigned long long *ticks) {
  half8_t a[4], b[4];
  uint32_t x = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
  for (int q = 0; q < 4; ++q)
    for (int v = 0; v < 8; ++v) {
      a[q][v] = (_Float16)operand(kind, x);
      b[q][v] = (_Float16)operand(kind, x);
    }
  floatx16 acc[16];
  for (int i = 0; i < 16; ++i)
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i & 3], b[(i >> 2) & 3], acc[i], 0, 0, 0);
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.f;
  for (int i = 0; i < 16; ++i)
    for (int v = 0; v < 16; ++v) s += acc[i][v];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = c1 - c0;
    ticks[2 * blockIdx.x + 1] = w1 - w0;
  }
}

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));     \
      return 1;                                                               \
    }                                                                         \
  } while (0)

int main() {
  int cus = 0, wall_khz = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0));
  const int blocks = cus, iters = 20000, reps = 3;
  float *sink = nullptr;
  unsigned long long *ticks = nullptr;
  CHECK(hipMalloc(&sink, sizeof(float) * blocks * 256));
  CHECK(hipMalloc(&ticks, sizeof(unsigned long long) * 2 * blocks));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const char *names[3] = {"const", "random", "nvfp4"};
  std::vector<unsigned long long> host(2 * blocks);
  for (int kind = 0; kind < 3; ++kind) {
    float ms = 0.f;
    for (int rep = 0; rep < reps; ++rep) {  // the last repetition runs at the settled clock
      CHECK(hipEventRecord(e0, 0));
      hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, 0, kind, iters, sink, ticks);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1, 0));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipEventElapsedTime(&ms, e0, e1));
    }
    CHECK(hipMemcpy(host.data(), ticks, sizeof(unsigned long long) * 2 * blocks, hipMemcpyDeviceToHost));
    double cyc = 0, wall = 0;
    for (int i = 0; i < blocks; ++i) {
      cyc += (double)host[2 * i];
      wall += (double)host[2 * i + 1];
    }
    const double mhz = cyc / (wall / (wall_khz * 1e3)) / 1e6;
    const double flops = 2.0 * 32 * 32 * 16 * 16.0 * iters * 4.0 * blocks;
    std::printf("{\"operands\": \"%s\", \"TFLOP/s\": %.1f, \"shader_MHz\": %.0f, \"cycles_per_mfma\": %.2f}\n",
                names[kind], flops / (ms * 1e-3) / 1e12, mhz, cyc / blocks / (16.0 * iters));
  }
  CHECK(hipFree(sink));
  CHECK(hipFree(ticks));
  return 0;
}
