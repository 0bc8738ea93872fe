// internal.hpp -- declarations shared by the library's translation units
// (kernels + launchers); not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

// Control words of one quantize workspace (4 KB, zero before first use).
// Two-pass path: the amax slots and the encode-pass completion counter are
// restored to zero by the last workgroup of each call.  Single-pass path: a
// grid barrier in two levels -- a workgroup adds one to arrive[blockIdx mod 8],
// the last arrival at a slot (it knows the launch's slot sizes) stores the
// slot back to zero and adds one to `top`, and the last of those stores `top`
// back to zero and publishes the next epoch in `release`.  Every call thus
// starts from zero counters whatever the grid size of the call before it.
// `release` counts completed single-pass calls (the current call's epoch);
// per-epoch-parity amax slots are cleared one call ahead.  The `fin` words
// count finished workgroups the same way, so that the last workgroup of the
// grid writes the tensor scale once every barrier wait of the call has either
// completed or expired.  Every word sits on its own 128-byte line so the
// atomics spread over memory channels.
struct QuantCtrl {
  uint32_t spin_limit; // single-pass: polls before a barrier wait gives up; 0 = the default (about 1 s)
  uint32_t done;       // two-pass: workgroups finished with the encode pass
  uint32_t timeout;    // single-pass: nonzero once a barrier wait expired (kept until the caller clears it)
  uint32_t pad0[29];
  struct alignas(128) Counter {
    unsigned long long v;
    uint32_t fin;
    uint32_t pad[29];
  } arrive[8], top, release;
  struct alignas(128) Slot {
    uint32_t v;
    uint32_t pad[31];
  } amax[2][8];
  // Two-pass: per-workgroup maxima go to slot blockIdx mod 8, so the atomics
  // of a pass that ends in one burst spread over four cache lines instead of
  // queueing on one word; readers take the max of the eight.
  struct alignas(64) Part {
    uint32_t v;
    uint32_t pad[15];
  } part[8];
  uint32_t pad1[32];
};
static_assert(sizeof(QuantCtrl) == 4096, "quantize control block is 4 KB");

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
  const float *clip;  // FP32 rows or dual views only: x <- clamp(x, -*clip, *clip) first (two passes)
};

// Several tensors quantized along their contiguous dimension with the same
// dtype and options.  Workspace: ctrl_seq serves the per-tensor fallback,
// ctrl_group the single-launch barrier, amax[j] (2 parities x 8 slots) the
// maxima of tensor j in that launch.
constexpr int kMaxGroup = 4;
struct QuantGroupProblem {
  int njobs;
  QuantProblem job[kMaxGroup];
  QuantCtrl *ctrl_seq, *ctrl_group;
  QuantCtrl::Slot (*amax[kMaxGroup])[8];
};
constexpr size_t kGroupWorkspace = 2 * sizeof(QuantCtrl) + kMaxGroup * 2 * 8 * sizeof(QuantCtrl::Slot);

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
  int tile_m, tile_n;  // 0, 0: automatic choice; otherwise a requested workgroup tile
  const float *cin;    // optional FP32 addend: y = fl(acc * s) + fl(beta * cin)
  int64_t ldcin, bstride_cin;
  float beta;
  const uint16_t *lr_t, *lr_l2;  // optional low-rank BF16 term lr_beta * T L2^T (batch 1)
  int64_t lr_r;
  float lr_beta;
  // Store the product transposed: element (m, n) at n * ldc + m, the addend
  // read the same way (FP32 output, ldc / ldcin / batch strides multiples of
  // 4 and C / cin 16-byte aligned; no low-rank term).
  bool c_transposed;
};

// Relative time of the automatic tile choice for an M x N product (units of
// tile area; lower is faster): lets a caller that may compute either C or
// C^T pick the orientation that fills the GPU better.
double gemm_tile_cost(int64_t M, int64_t N, int64_t K, int64_t batch);

// A symmetric product C = alpha s s A^ A^^T (+ beta cin), A^ [m][K] as both
// operands (the same codes, scales and tensor scale), FP32 C [m][m]: only the
// upper-triangle 256 x 256 tiles are computed, each split along K so that the
// items fill the GPU in one round, and a reduction adds the partial tiles in
// split order and writes both halves.  NVFP4_EUNSUPPORTED where the shape or
// the arguments do not allow it (the caller then runs launch_gemm);
// `part` holds gemm_symmetric_partial_bytes(m, K) bytes (0: not applicable).
size_t gemm_symmetric_partial_bytes(int64_t m, int64_t K);
nvfp4_status launch_gemm_symmetric(const GemmProblem &p, float *part, size_t part_bytes, hipStream_t stream);

// Exact order statistic of |x| (radix select): state->value = the element of
// rank `rank` (0-based, ascending by the bit pattern of |x|) of x [rows][cols]
// (row stride ld; cols and ld multiples of 4, x 16-byte aligned).  `hist`
// holds 4096 counters, zero on entry and on return.
struct SelectState {
  uint32_t prefix;
  float value;
  uint64_t rank;
  // the sampled bracket (see root.hip)
  uint32_t lo, hi;         // keys bracketing the rank, from a sorted sample
  uint32_t mode;           // 1: the bracket pass ran (its copy is used if it holds the rank); 0: it did not
  uint32_t overflow;       // the bracket held more keys than the compact buffer
  unsigned long long below;  // keys < lo
  uint32_t count;          // keys in [lo, hi], copied to the compact buffer
  uint32_t pad;
  uint64_t rank0;          // the target rank among all the keys
};
// `compact` holds `cap` keys (the bracket's copy).
nvfp4_status launch_abs_select(const float *x, int64_t rows, int64_t cols, int64_t ld, uint64_t rank,
                               SelectState *state, uint32_t *hist, uint32_t *compact, uint64_t cap,
                               hipStream_t stream);
// x = g / (||g||_F + 1e-7), with the norm from FP64 sums over 1024 fixed
// partials (partial: 1024 doubles) and *inv = fl32(1 / (||g|| + 1e-7)).
nvfp4_status launch_frobenius_normalize(const void *g, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                                        double *partial, float *inv, float *x, int64_t xld, hipStream_t stream);

// T = BF16_RNE(X L1^T): X [M][K] BF16 (row stride ldx, 16-byte aligned
// rows), L1 [r][K], T [M][r]; K % 16 == 0, r % 16 == 0, r <= 128.
nvfp4_status launch_lora_down(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint16_t *l1, int64_t r,
                              uint16_t *t, hipStream_t stream);

nvfp4_status launch_quantize(const QuantProblem &p, hipStream_t stream);
nvfp4_status launch_quantize_group(const QuantGroupProblem &p, hipStream_t stream);
// Both orientations of one input in one encode pass: `row` describes the
// input and the view along its columns, `col` the transposed view (its
// input fields are ignored); no transform; both views get one tensor scale.
nvfp4_status launch_quantize_dual(const QuantProblem &row, const QuantProblem &col, hipStream_t stream);
// Quantized optimizer state: the second moment's encode (square root, BF16
// block means into `means`, residual, transform, RNE; FP32 input, two passes)
// and the reconstruction of either state (`means` null: the first moment).
nvfp4_status launch_state_encode_second(const QuantProblem &p, uint16_t *means, hipStream_t stream);
nvfp4_status launch_state_decode(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                                 const uint16_t *means, float *out, int64_t rows, int64_t cols, int64_t ld,
                                 uint64_t rht_seed, hipStream_t stream);
nvfp4_status launch_gemm(const GemmProblem &p, hipStream_t stream);

}  // namespace nvfp4
