// internal.hpp -- declarations shared by the library's translation units
// (kernels + launchers); not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

// Control words of one quantize call, at the start of its workspace.  All
// words are zero between calls: the last workgroup of each call restores them.
struct QuantCtrl {
  uint32_t amax_bits;  // max |v| as FP32 bits, accumulated with atomicMax
  uint32_t done;       // workgroups finished with the encode pass
  uint32_t arrive;     // single-pass kernel: workgroups past the amax phase
  uint32_t depart;     // single-pass kernel: workgroups finished
  uint32_t timeout;    // single-pass kernel: a bounded wait expired
  uint32_t pad[59];
};
static_assert(sizeof(QuantCtrl) == 256, "control block is 256 bytes");

struct QuantProblem {
  const void *x;
  bool bf16;
  int64_t batch, rows, cols, ld, bstride;  // input view, elements
  bool along_rows;                          // transposing quantize
  bool sr, rht;
  uint64_t sr_seed, rht_seed;
  uint32_t sr_stream;
  uint8_t *codes, *scales;
  float *tensor_scale;
  QuantCtrl *ctrl;
};

struct GemmProblem {
  const uint8_t *a_codes, *a_scales;
  const float *a_st;
  const uint8_t *b_codes, *b_scales;
  const float *b_st;
  int64_t batch, M, N, K;
  void *c;
  bool c_bf16;
  int64_t ldc, bstride_c;
  float alpha;
};

nvfp4_status launch_quantize(const QuantProblem &p, hipStream_t stream);
nvfp4_status launch_gemm(const GemmProblem &p, hipStream_t stream);

}  // namespace nvfp4
