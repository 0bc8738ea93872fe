// api.hip -- the C ABI declared in include/nvfp4.h: argument validation (no
// HIP call before it passes), launch of the quantize / GEMM kernels, and the
// linear-layer driver (Fprop, Dgrad, Wgrad: six quantizations and three
// GEMMs on one stream, no host synchronisation).  Linear-projection training
// with NVFP4 GEMMs is the module "Full-Stack FP4 ..." treats in sections 1
// and 2.1; gradient tensors take stochastic rounding and the Wgrad operands
// the Hadamard mixing of section 2.2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/nvfp4.h"
#include "internal.hpp"

#define NVFP4_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using nvfp4::QuantCtrl;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxExtent = int64_t(1) << 40;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Validation of one quantized-view descriptor against an expected shape.
nvfp4_status check_view(const nvfp4_qtensor *q, int64_t batch, int64_t rows, int64_t cols) {
  if (!q) return NVFP4_EINVAL;
  if (q->batch != batch || q->rows != rows || q->cols != cols) return NVFP4_EINVAL;
  if (batch * rows * cols > 0 && (!q->codes || !q->scales)) return NVFP4_EINVAL;
  if (!q->tensor_scale) return NVFP4_EINVAL;
  if (!aligned(q->codes, 16) || !aligned(q->scales, 4) || !aligned(q->tensor_scale, 4))
    return NVFP4_EALIGN;
  return NVFP4_OK;
}

nvfp4_status validate_quantize(const void *x, int32_t x_dtype, int64_t batch, int64_t rows,
                               int64_t cols, int64_t ld, int64_t batch_stride, int32_t axis,
                               const nvfp4_quant_opts *opts, const nvfp4_qtensor *out,
                               const void *workspace, size_t workspace_bytes) {
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (axis != NVFP4_ALONG_COLS && axis != NVFP4_ALONG_ROWS) return NVFP4_EINVAL;
  if (opts) {
    if (opts->rounding != NVFP4_RNE && opts->rounding != NVFP4_SR) return NVFP4_EINVAL;
    if (opts->rht != 0 && opts->rht != 1) return NVFP4_EINVAL;
    if (opts->reserved != 0) return NVFP4_EINVAL;
  }
  if (batch < 0 || rows < 0 || cols < 0) return NVFP4_ESHAPE;
  if (batch > kMaxExtent || rows > kMaxExtent || cols > kMaxExtent) return NVFP4_ESHAPE;
  const int64_t contraction = axis == NVFP4_ALONG_COLS ? cols : rows;
  if (contraction % 16 != 0) return NVFP4_ESHAPE;
  const bool empty = batch == 0 || rows == 0 || cols == 0;
  if (!empty) {
    if (!x) return NVFP4_EINVAL;
    if (ld < cols) return NVFP4_ESHAPE;
    if (batch > 1 && batch_stride < rows * ld) return NVFP4_ESHAPE;
    if ((double)batch * (double)rows * (double)cols > 4.0e18) return NVFP4_ESHAPE;
  }
  const int64_t esize = x_dtype == NVFP4_F32 ? 4 : 2;
  if (!empty) {
    if (axis == NVFP4_ALONG_COLS &&
        (!aligned(x, 16) || (ld * esize) % 16 != 0 || (batch > 1 && (batch_stride * esize) % 16 != 0)))
      return NVFP4_EALIGN;
    if (axis == NVFP4_ALONG_ROWS && !aligned(x, (uintptr_t)esize)) return NVFP4_EALIGN;
  }
  const int64_t qr = axis == NVFP4_ALONG_COLS ? rows : cols;
  const int64_t qc = axis == NVFP4_ALONG_COLS ? cols : rows;
  nvfp4_status st = check_view(out, batch, qr, qc);
  if (st != NVFP4_OK) return st;
  if (!workspace || workspace_bytes < sizeof(QuantCtrl)) return NVFP4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_EALIGN;
  return NVFP4_OK;
}

nvfp4::QuantProblem make_quant(const void *x, bool bf16, int64_t batch, int64_t rows, int64_t cols,
                               int64_t ld, int64_t bstride, bool along_rows, const nvfp4_quant_opts *o,
                               const nvfp4_qtensor *out, void *ws) {
  nvfp4::QuantProblem p{};
  p.x = x;
  p.bf16 = bf16;
  p.batch = batch;
  p.rows = rows;
  p.cols = cols;
  p.ld = ld;
  p.bstride = bstride;
  p.along_rows = along_rows;
  p.sr = o && o->rounding == NVFP4_SR;
  p.rht = o && o->rht;
  p.sr_seed = o ? o->sr_seed : 0;
  p.rht_seed = o ? o->rht_seed : 0;
  p.sr_stream = o ? o->sr_stream : 0;
  p.codes = out->codes;
  p.scales = out->scales;
  p.tensor_scale = out->tensor_scale;
  p.ctrl = static_cast<QuantCtrl *>(ws);
  return p;
}

nvfp4_status validate_gemm(const nvfp4_qtensor *a, const nvfp4_qtensor *b, const void *c,
                           int32_t c_dtype, int64_t ldc, int64_t batch_stride_c) {
  if (!a || !b) return NVFP4_EINVAL;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (a->batch < 0 || a->rows < 0 || a->cols < 0 || b->rows < 0) return NVFP4_ESHAPE;
  if (a->cols % 16 != 0) return NVFP4_ESHAPE;
  if (a->batch != b->batch || a->cols != b->cols) return NVFP4_EINVAL;
  if (a->rows > kMaxExtent || b->rows > kMaxExtent || a->cols > kMaxExtent) return NVFP4_ESHAPE;
  nvfp4_status st = check_view(a, a->batch, a->rows, a->cols);
  if (st != NVFP4_OK) return st;
  st = check_view(b, b->batch, b->rows, b->cols);
  if (st != NVFP4_OK) return st;
  const int64_t M = a->rows, N = b->rows;
  if (a->batch * M * N > 0) {
    if (!c) return NVFP4_EINVAL;
    if (ldc < N) return NVFP4_ESHAPE;
    if (a->batch > 1 && batch_stride_c < M * ldc) return NVFP4_ESHAPE;
    if (!aligned(c, c_dtype == NVFP4_F32 ? 4 : 2)) return NVFP4_EALIGN;
    if (a->batch > 65535) return NVFP4_EUNSUPPORTED;
  }
  return NVFP4_OK;
}

nvfp4::GemmProblem make_gemm(const nvfp4_qtensor *a, const nvfp4_qtensor *b, void *c, int32_t c_dtype,
                             int64_t ldc, int64_t batch_stride_c, float alpha, int32_t tile_m = 0,
                             int32_t tile_n = 0) {
  nvfp4::GemmProblem p{};
  p.a_codes = a->codes;
  p.a_scales = a->scales;
  p.a_st = a->tensor_scale;
  p.b_codes = b->codes;
  p.b_scales = b->scales;
  p.b_st = b->tensor_scale;
  p.batch = a->batch;
  p.M = a->rows;
  p.N = b->rows;
  p.K = a->cols;
  p.c = c;
  p.c_bf16 = c_dtype == NVFP4_BF16;
  p.ldc = ldc;
  p.bstride_c = batch_stride_c;
  p.alpha = alpha;
  p.tile_m = tile_m;
  p.tile_n = tile_n;
  return p;
}

// Linear-driver workspace: six quantized views, each followed by its tensor
// scale and quantize control block, every region 256-byte aligned.
struct LinearLayout {
  size_t codes[6], scales[6], st[6], ctrl[6];
  int64_t rows[6], cols[6];
  size_t total;
};

LinearLayout linear_layout(int64_t M, int64_t N, int64_t K) {
  LinearLayout L{};
  const int64_t shapes[6][2] = {{M, K}, {N, K}, {M, N}, {K, N}, {N, M}, {K, M}};
  size_t off = 0;
  for (int i = 0; i < 6; ++i) {
    L.rows[i] = shapes[i][0];
    L.cols[i] = shapes[i][1];
    const size_t n = (size_t)shapes[i][0] * (size_t)shapes[i][1];
    L.codes[i] = off;
    off = round_up(off + n / 2, 256);
    L.scales[i] = off;
    off = round_up(off + n / 16, 256);
    L.st[i] = off;
    off += 256;
    L.ctrl[i] = off;
    off += sizeof(QuantCtrl);
  }
  L.total = off;
  return L;
}

// Scratch of nvfp4_quantize_noalloc: one quantize control block (4 KiB) in
// the library's own device memory, one copy per GPU, zero when the module is
// loaded.  Every call leaves it ready for the next (the control block's own
// rule), so nothing is cleared between calls.  Host code never uses the
// array's name as an address: each device's copy is looked up once with
// hipGetSymbolAddress, with that device current, and kept.
constexpr size_t kScratchBytes = sizeof(QuantCtrl);
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

nvfp4_status scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return NVFP4_EHIP;
  if (dev >= kMaxDevices) return NVFP4_EUNSUPPORTED;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Concurrent first calls on one device look up the same address.
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return NVFP4_EHIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return NVFP4_OK;
}

// Attention dS workspace: the two quantized views of dS (along the keys,
// [bh][sq][sk], and along the queries, [bh][sk][sq]) with their tensor-scale
// slots, then one quantize control block; every region 256-byte aligned.
struct AttnLayout {
  size_t codes[2], scales[2], st[2], ctrl;
  size_t total;
};

AttnLayout attn_layout(int64_t bh, int64_t sq, int64_t sk) {
  AttnLayout L{};
  const size_t n = (size_t)bh * (size_t)sq * (size_t)sk;
  size_t off = 0;
  for (int i = 0; i < 2; ++i) {
    L.codes[i] = off;
    off = round_up(off + n / 2, 256);
    L.scales[i] = off;
    off = round_up(off + n / 16, 256);
    L.st[i] = off;
    off += 256;
  }
  L.ctrl = off;
  L.total = off + sizeof(QuantCtrl);
  return L;
}

}  // namespace

NVFP4_EXPORT const char *nvfp4_status_string(int32_t status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument";
    case NVFP4_ESHAPE: return "unsupported shape (contraction length must be a multiple of 16)";
    case NVFP4_EALIGN: return "misaligned pointer or stride";
    case NVFP4_EUNSUPPORTED: return "unsupported request";
    case NVFP4_EHIP: return "HIP launch failed";
    case NVFP4_EWORKSPACE: return "workspace missing or too small";
    case NVFP4_ETIMEOUT: return "a single-pass quantize gave up waiting at its grid barrier (results unreliable)";
    default: return "unknown status";
  }
}

NVFP4_EXPORT int32_t nvfp4_version(void) { return (1 << 16) | 2; }

NVFP4_EXPORT size_t nvfp4_quantize_workspace_size(void) { return sizeof(QuantCtrl); }

NVFP4_EXPORT nvfp4_status nvfp4_quantize(const void *x, int32_t x_dtype, int64_t batch, int64_t rows,
                                         int64_t cols, int64_t ld, int64_t batch_stride, int32_t axis,
                                         const nvfp4_quant_opts *opts, const nvfp4_qtensor *out,
                                         void *workspace, size_t workspace_bytes, void *stream) {
  nvfp4_status st = validate_quantize(x, x_dtype, batch, rows, cols, ld, batch_stride, axis, opts, out,
                                      workspace, workspace_bytes);
  if (st != NVFP4_OK) return st;
  const nvfp4::QuantProblem p = make_quant(x, x_dtype == NVFP4_BF16, batch, rows, cols, ld, batch_stride,
                                           axis == NVFP4_ALONG_ROWS, opts, out, workspace);
  return nvfp4::launch_quantize(p, static_cast<hipStream_t>(stream));
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize_noalloc(const void *x, int32_t x_dtype, int64_t batch, int64_t rows,
                                                 int64_t cols, int64_t ld, int64_t batch_stride, int32_t axis,
                                                 const nvfp4_quant_opts *opts, const nvfp4_qtensor *out,
                                                 void *stream) {
  // Arguments first, as for nvfp4_quantize (the workspace check is passed a
  // stand-in of the scratch's size; no HIP call happens before this).
  static_assert(kScratchBytes >= sizeof(QuantCtrl), "the scratch holds one control block");
  nvfp4_status st = validate_quantize(x, x_dtype, batch, rows, cols, ld, batch_stride, axis, opts, out,
                                      reinterpret_cast<const void *>(uintptr_t(256)), kScratchBytes);
  if (st != NVFP4_OK) return st;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != NVFP4_OK) return st;
  const nvfp4::QuantProblem p = make_quant(x, x_dtype == NVFP4_BF16, batch, rows, cols, ld, batch_stride,
                                           axis == NVFP4_ALONG_ROWS, opts, out, ws);
  return nvfp4::launch_quantize(p, static_cast<hipStream_t>(stream));
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize_dual(const void *x, int32_t x_dtype, int64_t batch, int64_t rows,
                                              int64_t cols, int64_t ld, int64_t batch_stride,
                                              const nvfp4_quant_opts *row_opts, const nvfp4_qtensor *row_out,
                                              const nvfp4_quant_opts *col_opts, const nvfp4_qtensor *col_out,
                                              void *workspace, size_t workspace_bytes, void *stream) {
  // Each view is validated as its single-orientation call would be; both
  // extents must then be multiples of 16, and neither view may ask for the
  // transform (it would make the two views' maxima differ).
  // The transposed view as for ALONG_ROWS (x aligned to its element size,
  // rows % 16 == 0), then the view along the columns: its options, cols %
  // 16 == 0 and its descriptor.
  nvfp4_status st = validate_quantize(x, x_dtype, batch, rows, cols, ld, batch_stride, NVFP4_ALONG_ROWS, col_opts,
                                      col_out, workspace, workspace_bytes);
  if (st != NVFP4_OK) return st;
  if (row_opts) {
    if (row_opts->rounding != NVFP4_RNE && row_opts->rounding != NVFP4_SR) return NVFP4_EINVAL;
    if (row_opts->rht != 0 && row_opts->rht != 1) return NVFP4_EINVAL;
    if (row_opts->reserved != 0) return NVFP4_EINVAL;
  }
  if (cols % 16 != 0) return NVFP4_ESHAPE;
  st = check_view(row_out, batch, rows, cols);
  if (st != NVFP4_OK) return st;
  if ((row_opts && row_opts->rht) || (col_opts && col_opts->rht)) return NVFP4_EUNSUPPORTED;
  const nvfp4::QuantProblem pr = make_quant(x, x_dtype == NVFP4_BF16, batch, rows, cols, ld, batch_stride, false,
                                            row_opts, row_out, workspace);
  const nvfp4::QuantProblem pc = make_quant(x, x_dtype == NVFP4_BF16, batch, rows, cols, ld, batch_stride, true,
                                            col_opts, col_out, workspace);
  return nvfp4::launch_quantize_dual(pr, pc, static_cast<hipStream_t>(stream));
}

NVFP4_EXPORT size_t nvfp4_qadamw_workspace_size(void) { return 2 * sizeof(QuantCtrl); }

namespace {
nvfp4_status validate_state(const nvfp4_qadamw_state *st, int64_t rows, int64_t cols) {
  if (!st) return NVFP4_EINVAL;
  nvfp4_status r = check_view(&st->m, 1, rows, cols);
  if (r != NVFP4_OK) return r;
  r = check_view(&st->v, 1, rows, cols);
  if (r != NVFP4_OK) return r;
  if (rows * cols > 0 && !st->v_means) return NVFP4_EINVAL;
  if (!aligned(st->v_means, 2)) return NVFP4_EALIGN;
  return NVFP4_OK;
}
}  // namespace

NVFP4_EXPORT nvfp4_status nvfp4_qadamw_encode(const float *m, const float *v, int64_t rows, int64_t cols, int64_t ld,
                                              uint64_t rht_seed, uint64_t sr_seed, uint32_t sr_stream,
                                              const nvfp4_qadamw_state *state, void *workspace,
                                              size_t workspace_bytes, void *stream) {
  if (rows < 0 || cols < 0 || rows > kMaxExtent || cols > kMaxExtent || cols % 16) return NVFP4_ESHAPE;
  if (rows * cols > 0 && (!m || !v)) return NVFP4_EINVAL;
  if (rows * cols > 0 && (ld < cols || !aligned(m, 16) || !aligned(v, 16) || (ld * 4) % 16)) {
    return ld < cols ? NVFP4_ESHAPE : NVFP4_EALIGN;
  }
  nvfp4_status r = validate_state(state, rows, cols);
  if (r != NVFP4_OK) return r;
  if (!workspace || workspace_bytes < 2 * sizeof(QuantCtrl)) return NVFP4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_EALIGN;
  QuantCtrl *ctrl = static_cast<QuantCtrl *>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // First moment: the transform, then stochastic rounding.
  const nvfp4_quant_opts mo{NVFP4_SR, 1, sr_seed, rht_seed, sr_stream, 0u};
  r = nvfp4::launch_quantize(make_quant(m, false, 1, rows, cols, ld, rows * ld, false, &mo, &state->m, ctrl), s);
  if (r != NVFP4_OK) return r;
  // Second moment: square root, block means, residual, the transform, RNE.
  const nvfp4_quant_opts vo{NVFP4_RNE, 1, 0, rht_seed, 0u, 0u};
  return nvfp4::launch_state_encode_second(make_quant(v, false, 1, rows, cols, ld, rows * ld, false, &vo, &state->v,
                                                      ctrl + 1),
                                           state->v_means, s);
}

NVFP4_EXPORT nvfp4_status nvfp4_qadamw_decode(const nvfp4_qadamw_state *state, uint64_t rht_seed, float *m, float *v,
                                              int64_t ld, void *stream) {
  if (!state) return NVFP4_EINVAL;
  const int64_t rows = state->m.rows, cols = state->m.cols;
  if (rows < 0 || cols < 0 || cols % 16 || rows > kMaxExtent || cols > kMaxExtent) return NVFP4_ESHAPE;
  nvfp4_status r = validate_state(state, rows, cols);
  if (r != NVFP4_OK) return r;
  if (rows * cols > 0) {
    if (!m || !v) return NVFP4_EINVAL;
    if (ld < cols) return NVFP4_ESHAPE;
    if (!aligned(m, 16) || !aligned(v, 16) || (ld * 4) % 16) return NVFP4_EALIGN;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  r = nvfp4::launch_state_decode(state->m.codes, state->m.scales, state->m.tensor_scale, nullptr, m, rows, cols, ld,
                                 rht_seed, s);
  if (r != NVFP4_OK) return r;
  return nvfp4::launch_state_decode(state->v.codes, state->v.scales, state->v.tensor_scale, state->v_means, v, rows,
                                    cols, ld, rht_seed, s);
}

NVFP4_EXPORT size_t nvfp4_quantize_group_workspace_size(void) { return nvfp4::kGroupWorkspace; }

NVFP4_EXPORT nvfp4_status nvfp4_quantize_group(const nvfp4_quant_job *jobs, int32_t njobs, int32_t x_dtype,
                                               const nvfp4_quant_opts *opts, void *workspace,
                                               size_t workspace_bytes, void *stream) {
  if (!jobs || njobs < 1 || njobs > nvfp4::kMaxGroup) return NVFP4_EINVAL;
  for (int i = 0; i < njobs; ++i) {
    const nvfp4_quant_job &j = jobs[i];
    const nvfp4_status st = validate_quantize(j.x, x_dtype, j.batch, j.rows, j.cols, j.ld, j.batch_stride,
                                              NVFP4_ALONG_COLS, opts, &j.out, workspace, workspace_bytes);
    if (st != NVFP4_OK) return st;
  }
  if (workspace_bytes < nvfp4::kGroupWorkspace) return NVFP4_EWORKSPACE;
  nvfp4::QuantGroupProblem p{};
  p.njobs = njobs;
  for (int i = 0; i < njobs; ++i) {
    const nvfp4_quant_job &j = jobs[i];
    p.job[i] = make_quant(j.x, x_dtype == NVFP4_BF16, j.batch, j.rows, j.cols, j.ld, j.batch_stride, false, opts,
                          &j.out, workspace);
  }
  uint8_t *base = static_cast<uint8_t *>(workspace);
  p.ctrl_seq = reinterpret_cast<QuantCtrl *>(base);
  p.ctrl_group = reinterpret_cast<QuantCtrl *>(base + sizeof(QuantCtrl));
  for (int i = 0; i < nvfp4::kMaxGroup; ++i)
    p.amax[i] = reinterpret_cast<QuantCtrl::Slot(*)[8]>(base + 2 * sizeof(QuantCtrl) +
                                                        i * 2 * 8 * sizeof(QuantCtrl::Slot));
  return nvfp4::launch_quantize_group(p, static_cast<hipStream_t>(stream));
}

NVFP4_EXPORT nvfp4_status nvfp4_gemm(const nvfp4_qtensor *a, const nvfp4_qtensor *b, void *c, int32_t c_dtype,
                                     int64_t ldc, int64_t batch_stride_c, float alpha, void *stream) {
  nvfp4_status st = validate_gemm(a, b, c, c_dtype, ldc, batch_stride_c);
  if (st != NVFP4_OK) return st;
  return nvfp4::launch_gemm(make_gemm(a, b, c, c_dtype, ldc, batch_stride_c, alpha),
                            static_cast<hipStream_t>(stream));
}

NVFP4_EXPORT nvfp4_status nvfp4_gemm_ex(const nvfp4_qtensor *a, const nvfp4_qtensor *b, void *c, int32_t c_dtype,
                                        int64_t ldc, int64_t batch_stride_c, float alpha, int32_t tile_m,
                                        int32_t tile_n, void *stream) {
  nvfp4_status st = validate_gemm(a, b, c, c_dtype, ldc, batch_stride_c);
  if (st != NVFP4_OK) return st;
  if (tile_m < 0 || tile_n < 0 || (tile_m == 0) != (tile_n == 0)) return NVFP4_EINVAL;
  return nvfp4::launch_gemm(make_gemm(a, b, c, c_dtype, ldc, batch_stride_c, alpha, tile_m, tile_n),
                            static_cast<hipStream_t>(stream));
}

NVFP4_EXPORT nvfp4_status nvfp4_gemm_axpby(const nvfp4_qtensor *a, const nvfp4_qtensor *b, void *c, int32_t c_dtype,
                                           int64_t ldc, int64_t batch_stride_c, float alpha, const float *c_in,
                                           int64_t ldc_in, int64_t batch_stride_c_in, float beta, void *stream) {
  nvfp4_status st = validate_gemm(a, b, c, c_dtype, ldc, batch_stride_c);
  if (st != NVFP4_OK) return st;
  const int64_t M = a->rows, N = b->rows;
  if (a->batch * M * N > 0) {
    if (!c_in) return NVFP4_EINVAL;
    if (ldc_in < N) return NVFP4_ESHAPE;
    if (a->batch > 1 && batch_stride_c_in < M * ldc_in) return NVFP4_ESHAPE;
    if (!aligned(c_in, 4)) return NVFP4_EALIGN;
    // In place is allowed only as the very same array.
    if (static_cast<const void *>(c_in) == c && (c_dtype != NVFP4_F32 || ldc_in != ldc ||
                                                 (a->batch > 1 && batch_stride_c_in != batch_stride_c)))
      return NVFP4_EINVAL;
  }
  nvfp4::GemmProblem p = make_gemm(a, b, c, c_dtype, ldc, batch_stride_c, alpha);
  p.cin = c_in;
  p.ldcin = ldc_in;
  p.bstride_cin = batch_stride_c_in;
  p.beta = beta;
  return nvfp4::launch_gemm(p, static_cast<hipStream_t>(stream));
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize_workspace_check(const void *workspace, size_t workspace_bytes,
                                                         void *stream) {
  if (!workspace || workspace_bytes < sizeof(QuantCtrl)) return NVFP4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_EALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // The control blocks a workspace of this size holds: the per-tensor one,
  // and for a group workspace the single-launch one after it.
  const int nblocks = workspace_bytes >= nvfp4::kGroupWorkspace ? 2 : 1;
  uint32_t words[2] = {0u, 0u};
  for (int i = 0; i < nblocks; ++i) {
    const QuantCtrl *c = static_cast<const QuantCtrl *>(workspace) + i;
    if (hipMemcpyAsync(&words[i], &c->timeout, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
      return NVFP4_EHIP;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return NVFP4_EHIP;
  return (words[0] | words[1]) ? NVFP4_ETIMEOUT : NVFP4_OK;
}

NVFP4_EXPORT size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxExtent || N > kMaxExtent || K > kMaxExtent) return 0;
  return linear_layout(M, N, K).total;
}

NVFP4_EXPORT nvfp4_status nvfp4_linear_view(void *workspace, size_t workspace_bytes, int64_t M, int64_t N,
                                            int64_t K, int32_t which, nvfp4_qtensor *out) {
  if (!workspace || !out || which < 0 || which > 5) return NVFP4_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || M % 16 || N % 16 || K % 16) return NVFP4_ESHAPE;
  if (M > kMaxExtent || N > kMaxExtent || K > kMaxExtent) return NVFP4_ESHAPE;
  const LinearLayout L = linear_layout(M, N, K);
  if (workspace_bytes < L.total) return NVFP4_EWORKSPACE;
  uint8_t *base = static_cast<uint8_t *>(workspace);
  out->codes = base + L.codes[which];
  out->scales = base + L.scales[which];
  out->tensor_scale = reinterpret_cast<float *>(base + L.st[which]);
  out->batch = 1;
  out->rows = L.rows[which];
  out->cols = L.cols[which];
  return NVFP4_OK;
}

NVFP4_EXPORT size_t nvfp4_attention_ds_workspace_size(int64_t bh, int64_t sq, int64_t sk) {
  if (bh <= 0 || sq <= 0 || sk <= 0 || bh > kMaxExtent || sq > kMaxExtent || sk > kMaxExtent) return 0;
  return attn_layout(bh, sq, sk).total;
}

NVFP4_EXPORT nvfp4_status nvfp4_attention_ds_grads(const void *ds, int32_t ds_dtype, const nvfp4_qtensor *q_seq,
                                                   const nvfp4_qtensor *k_seq, void *dq, void *dk, int32_t out_dtype,
                                                   int64_t bh, int64_t sq, int64_t sk, int64_t d, float alpha,
                                                   const nvfp4_attn_cfg *cfg, void *workspace,
                                                   size_t workspace_bytes, void *stream) {
  if (!ds || !q_seq || !k_seq || !dq || !dk || !cfg) return NVFP4_EINVAL;
  if (ds_dtype != NVFP4_F32 && ds_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (cfg->ds_rounding != NVFP4_RNE && cfg->ds_rounding != NVFP4_SR) return NVFP4_EINVAL;
  if (cfg->reserved != 0) return NVFP4_EINVAL;
  if (bh <= 0 || sq <= 0 || sk <= 0 || d <= 0 || sq % 16 || sk % 16 || d % 16) return NVFP4_ESHAPE;
  if (bh > 65535 || sq > kMaxExtent || sk > kMaxExtent || d > kMaxExtent) return NVFP4_ESHAPE;
  nvfp4_status st = check_view(q_seq, bh, d, sq);
  if (st != NVFP4_OK) return st;
  st = check_view(k_seq, bh, d, sk);
  if (st != NVFP4_OK) return st;
  if (!aligned(ds, 16) || !aligned(dq, 16) || !aligned(dk, 16)) return NVFP4_EALIGN;
  const AttnLayout L = attn_layout(bh, sq, sk);
  if (!workspace || workspace_bytes < L.total) return NVFP4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_EALIGN;
  uint8_t *base = static_cast<uint8_t *>(workspace);
  nvfp4_qtensor ds_row{base + L.codes[0], base + L.scales[0], reinterpret_cast<float *>(base + L.st[0]), bh, sq, sk};
  nvfp4_qtensor ds_col{base + L.codes[1], base + L.scales[1], reinterpret_cast<float *>(base + L.st[1]), bh, sk, sq};
  nvfp4_quant_opts row_o{cfg->ds_rounding, 0, cfg->sr_seed, 0, 4u, 0u};
  nvfp4_quant_opts col_o{cfg->ds_rounding, 0, cfg->sr_seed, 0, 5u, 0u};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const nvfp4::QuantProblem pr = make_quant(ds, ds_dtype == NVFP4_BF16, bh, sq, sk, sk, sq * sk, false, &row_o,
                                            &ds_row, base + L.ctrl);
  const nvfp4::QuantProblem pc = make_quant(ds, ds_dtype == NVFP4_BF16, bh, sq, sk, sk, sq * sk, true, &col_o,
                                            &ds_col, base + L.ctrl);
  st = nvfp4::launch_quantize_dual(pr, pc, s);
  if (st != NVFP4_OK) return st;
  // dQ = alpha dS K: dS along the keys, K^T along the keys;  dK = alpha dS^T Q: dS^T and Q^T along the queries.
  st = nvfp4::launch_gemm(make_gemm(&ds_row, k_seq, dq, out_dtype, d, sq * d, alpha), s);
  if (st != NVFP4_OK) return st;
  return nvfp4::launch_gemm(make_gemm(&ds_col, q_seq, dk, out_dtype, d, sk * d, alpha), s);
}

NVFP4_EXPORT nvfp4_status nvfp4_linear_fwd_bwd(const void *x, const void *w, const void *dy, void *y,
                                               void *dx, void *dw, int64_t M, int64_t N, int64_t K,
                                               const nvfp4_linear_cfg *cfg, void *workspace,
                                               size_t workspace_bytes, void *stream) {
  if (!cfg || !x || !w || !dy || !y || !dx || !dw) return NVFP4_EINVAL;
  if (cfg->dw_dtype != NVFP4_F32 && cfg->dw_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || M % 16 || N % 16 || K % 16) return NVFP4_ESHAPE;
  if (M > kMaxExtent || N > kMaxExtent || K > kMaxExtent) return NVFP4_ESHAPE;
  for (const void *p : {x, w, dy, static_cast<const void *>(y), static_cast<const void *>(dx),
                        static_cast<const void *>(dw)})
    if (!aligned(p, 16)) return NVFP4_EALIGN;
  const LinearLayout L = linear_layout(M, N, K);
  if (!workspace || workspace_bytes < L.total) return NVFP4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_EALIGN;

  uint8_t *base = static_cast<uint8_t *>(workspace);
  nvfp4_qtensor v[6];
  for (int i = 0; i < 6; ++i) {
    v[i].codes = base + L.codes[i];
    v[i].scales = base + L.scales[i];
    v[i].tensor_scale = reinterpret_cast<float *>(base + L.st[i]);
    v[i].batch = 1;
    v[i].rows = L.rows[i];
    v[i].cols = L.cols[i];
  }
  auto ctrl = [&](int i) { return static_cast<void *>(base + L.ctrl[i]); };
  const hipStream_t s = static_cast<hipStream_t>(stream);
  nvfp4_quant_opts rne{};
  nvfp4_quant_opts dy_row{NVFP4_SR, 0, cfg->sr_seed, cfg->rht_seed, 1u, 0u};
  nvfp4_quant_opts dy_col{NVFP4_SR, 1, cfg->sr_seed, cfg->rht_seed, 2u, 0u};
  nvfp4_quant_opts x_col{cfg->wgrad_sr_x ? NVFP4_SR : NVFP4_RNE, 1, cfg->sr_seed, cfg->rht_seed, 3u, 0u};

  struct Q {
    const void *src;
    int64_t rows, cols;
    bool along_rows;
    const nvfp4_quant_opts *o;
  } qs[6] = {{x, M, K, false, &rne},   {w, N, K, false, &rne},  {dy, M, N, false, &dy_row},
             {w, N, K, true, &rne},    {dy, M, N, true, &dy_col}, {x, M, K, true, &x_col}};
  const struct {
    int a, b;
    void *c;
    int32_t dtype;
    int64_t ldc;
  } gs[3] = {{0, 1, y, NVFP4_BF16, N}, {2, 3, dx, NVFP4_BF16, K}, {4, 5, dw, cfg->dw_dtype, K}};

  for (int gi = 0; gi < 3; ++gi) {
    for (int qi : {gs[gi].a, gs[gi].b}) {
      const Q &q = qs[qi];
      const nvfp4::QuantProblem p =
          make_quant(q.src, true, 1, q.rows, q.cols, q.cols, q.rows * q.cols, q.along_rows, q.o, &v[qi], ctrl(qi));
      const nvfp4_status st = nvfp4::launch_quantize(p, s);
      if (st != NVFP4_OK) return st;
    }
    const nvfp4_status st =
        nvfp4::launch_gemm(make_gemm(&v[gs[gi].a], &v[gs[gi].b], gs[gi].c, gs[gi].dtype, gs[gi].ldc, 0, 1.0f), s);
    if (st != NVFP4_OK) return st;
  }
  return NVFP4_OK;
}

// ---------------------------------------------------------------------------
// Newton-Schulz orthogonalization with every matrix product in NVFP4
// ("Full-Stack FP4 ...", section 2.3, Q-Root).
// ---------------------------------------------------------------------------

namespace {

// Workspace: three quantize control blocks, three select states (X, A, B)
// and their shared 4096-counter histogram and compact buffer, the normalization partials, the second iterate
// buffer, A and B in FP32, the partial tiles of the symmetric products, and
// the four quantized views; 256-byte regions.
struct NsLayout {
  size_t ctrl[3], sel[3], hist, compact, partial, inv, xbuf, a, b, sym, sym_bytes;
  uint64_t cap;  // keys the select's compact buffer holds
  size_t codes[4], scales[4], st[4];
  int64_t rows[4], cols[4];
  size_t total;
};

NsLayout ns_layout(int64_t m, int64_t n) {
  NsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  for (int i = 0; i < 3; ++i) L.ctrl[i] = take(sizeof(QuantCtrl));
  for (int i = 0; i < 3; ++i) L.sel[i] = take(sizeof(nvfp4::SelectState));
  L.hist = take(4096 * sizeof(uint32_t));
  // the select's bracket copy: a sixteenth of the larger operand (the
  // bracket holds about 5% of it; more falls back to the full passes)
  L.cap = ((uint64_t)m * (uint64_t)(n > m ? n : m)) / 16 + 1024;
  L.compact = take(L.cap * sizeof(uint32_t));
  L.partial = take(1024 * sizeof(double));
  L.inv = take(sizeof(float));
  L.xbuf = take((size_t)m * (size_t)n * 4);
  L.a = take((size_t)m * (size_t)m * 4);
  L.b = take((size_t)m * (size_t)m * 4);
  L.sym_bytes = std::max(nvfp4::gemm_symmetric_partial_bytes(m, n), nvfp4::gemm_symmetric_partial_bytes(m, m));
  L.sym = take(L.sym_bytes);
  const int64_t shapes[4][2] = {{m, n}, {n, m}, {m, m}, {m, m}};
  for (int i = 0; i < 4; ++i) {
    L.rows[i] = shapes[i][0];
    L.cols[i] = shapes[i][1];
    const size_t e = (size_t)shapes[i][0] * (size_t)shapes[i][1];
    L.codes[i] = take(e / 2);
    L.scales[i] = take(e / 16);
    L.st[i] = take(sizeof(float));
  }
  L.total = off;
  return L;
}

nvfp4_qtensor ns_view(uint8_t *base, const NsLayout &L, int i) {
  nvfp4_qtensor q{};
  q.codes = base + L.codes[i];
  q.scales = base + L.scales[i];
  q.tensor_scale = reinterpret_cast<float *>(base + L.st[i]);
  q.batch = 1;
  q.rows = L.rows[i];
  q.cols = L.cols[i];
  return q;
}

bool ns_shape_ok(int64_t m, int64_t n) {
  return m > 0 && n > 0 && m % 16 == 0 && n % 16 == 0 && m <= (int64_t(1) << 20) && n <= (int64_t(1) << 20) &&
         (double)m * (double)n < 4.0e9;
}

// 0-based rank of the q-quantile of N values: the ceil(q N)-th smallest.
uint64_t quantile_rank(double q, uint64_t n) {
  double k = std::ceil(q * (double)n);
  if (k < 1.0) k = 1.0;
  if (k > (double)n) k = (double)n;
  return (uint64_t)k - 1;
}

}  // namespace

NVFP4_EXPORT size_t nvfp4_ns_workspace_size(int64_t m, int64_t n) {
  if (!ns_shape_ok(m, n)) return 0;
  return ns_layout(m, n).total;
}

NVFP4_EXPORT nvfp4_status nvfp4_ns_internals(void *workspace, size_t workspace_bytes, int64_t m, int64_t n,
                                             nvfp4_ns_state *out) {
  if (!workspace || !out) return NVFP4_EINVAL;
  if (!ns_shape_ok(m, n)) return NVFP4_ESHAPE;
  const NsLayout L = ns_layout(m, n);
  if (workspace_bytes < L.total) return NVFP4_EWORKSPACE;
  uint8_t *base = static_cast<uint8_t *>(workspace);
  out->x_prev = reinterpret_cast<float *>(base + L.xbuf);
  out->a = reinterpret_cast<float *>(base + L.a);
  out->b = reinterpret_cast<float *>(base + L.b);
  for (int i = 0; i < 3; ++i)
    out->clip[i] = &reinterpret_cast<nvfp4::SelectState *>(base + L.sel[i])->value;
  out->inv_norm = reinterpret_cast<float *>(base + L.inv);
  for (int i = 0; i < 4; ++i) out->view[i] = ns_view(base, L, i);
  return NVFP4_OK;
}

NVFP4_EXPORT nvfp4_status nvfp4_ns_orthogonalize(const void *g, int32_t g_dtype, int64_t m, int64_t n, int64_t ldg,
                                                 const float *coeffs, int32_t steps, const nvfp4_ns_cfg *cfg,
                                                 float *x, int64_t ldx, void *workspace, size_t workspace_bytes,
                                                 void *stream) {
  if (!g || !x || !cfg || (steps > 0 && !coeffs)) return NVFP4_EINVAL;
  if (g_dtype != NVFP4_F32 && g_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (steps < 0 || steps > 64) return NVFP4_EINVAL;
  if (cfg->clip_mask > 7u || cfg->product > 2u) return NVFP4_EINVAL;
  if (cfg->clip_mask && !(cfg->clip_quantile > 0.0 && cfg->clip_quantile <= 1.0)) return NVFP4_EINVAL;
  if (!ns_shape_ok(m, n)) return NVFP4_ESHAPE;
  if (ldg < n || ldx < n) return NVFP4_ESHAPE;
  const size_t gsz = g_dtype == NVFP4_F32 ? 4 : 2;
  if (!aligned(g, 4 * gsz) || ldg % 4 || !aligned(x, 16) || ldx % 4) return NVFP4_EALIGN;
  const NsLayout L = ns_layout(m, n);
  if (!workspace || workspace_bytes < L.total) return NVFP4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_EALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *base = static_cast<uint8_t *>(workspace);
  float *xbuf = reinterpret_cast<float *>(base + L.xbuf);
  float *A = reinterpret_cast<float *>(base + L.a);
  float *B = reinterpret_cast<float *>(base + L.b);
  auto sel = [&](int i) { return reinterpret_cast<nvfp4::SelectState *>(base + L.sel[i]); };
  uint32_t *hist = reinterpret_cast<uint32_t *>(base + L.hist);
  uint32_t *compact = reinterpret_cast<uint32_t *>(base + L.compact);
  const nvfp4_qtensor vX = ns_view(base, L, 0), vXT = ns_view(base, L, 1), vA = ns_view(base, L, 2),
                      vB = ns_view(base, L, 3);
  // The iterates alternate so that the last one lands in x.
  float *P[2];
  int64_t ldp[2];
  P[steps % 2] = x;
  ldp[steps % 2] = ldx;
  P[(steps + 1) % 2] = xbuf;
  ldp[(steps + 1) % 2] = n;
  nvfp4_status r = nvfp4::launch_frobenius_normalize(g, g_dtype == NVFP4_BF16, m, n, ldg,
                                                     reinterpret_cast<double *>(base + L.partial),
                                                     reinterpret_cast<float *>(base + L.inv), P[0], ldp[0], s);
  if (r != NVFP4_OK) return r;
  const nvfp4_quant_opts rne{NVFP4_RNE, 0, 0, 0, 0u, 0u};
  const bool transposed = cfg->product == 2u || (cfg->product == 0u && nvfp4::gemm_tile_cost(n, m, m, 1) <
                                                                            nvfp4::gemm_tile_cost(m, n, m, 1));
  for (int k = 0; k < steps; ++k) {
    float *Xc = P[k % 2], *Xn = P[(k + 1) % 2];
    const int64_t ldc_ = ldp[k % 2], ldn = ldp[(k + 1) % 2];
    const float ca = coeffs[3 * k], cb = coeffs[3 * k + 1], cc = coeffs[3 * k + 2];
    // X: clip value, then both orientations from one read.
    const float *clip_x = nullptr;
    if (cfg->clip_mask & 1u) {
      r = nvfp4::launch_abs_select(Xc, m, n, ldc_, quantile_rank(cfg->clip_quantile, (uint64_t)(m * n)), sel(0),
                                   hist, compact, L.cap, s);
      if (r != NVFP4_OK) return r;
      clip_x = &sel(0)->value;
    }
    nvfp4::QuantProblem qx = make_quant(Xc, false, 1, m, n, ldc_, m * ldc_, false, &rne, &vX, base + L.ctrl[0]);
    qx.clip = clip_x;
    nvfp4::QuantProblem qxt = make_quant(Xc, false, 1, m, n, ldc_, m * ldc_, true, &rne, &vXT, base + L.ctrl[0]);
    r = nvfp4::launch_quantize_dual(qx, qxt, s);
    if (r != NVFP4_OK) return r;
    // A = X X^T (symmetric: the upper triangle split along K, where it applies)
    float *part = reinterpret_cast<float *>(base + L.sym);
    const nvfp4::GemmProblem pa = make_gemm(&vX, &vX, A, NVFP4_F32, m, m * m, 1.0f);
    r = nvfp4::launch_gemm_symmetric(pa, part, L.sym_bytes, s);
    if (r == NVFP4_EUNSUPPORTED) r = nvfp4::launch_gemm(pa, s);
    if (r != NVFP4_OK) return r;
    const float *clip_a = nullptr;
    if (cfg->clip_mask & 2u) {
      r = nvfp4::launch_abs_select(A, m, m, m, quantile_rank(cfg->clip_quantile, (uint64_t)(m * m)), sel(1), hist, compact, L.cap, s);
      if (r != NVFP4_OK) return r;
      clip_a = &sel(1)->value;
    }
    nvfp4::QuantProblem qa = make_quant(A, false, 1, m, m, m, m * m, false, &rne, &vA, base + L.ctrl[1]);
    qa.clip = clip_a;
    r = nvfp4::launch_quantize(qa, s);
    if (r != NVFP4_OK) return r;
    // B = c A A^T + b A  (A is symmetric)
    nvfp4::GemmProblem pb = make_gemm(&vA, &vA, B, NVFP4_F32, m, m * m, cc);
    pb.cin = A;
    pb.ldcin = m;
    pb.bstride_cin = m * m;
    pb.beta = cb;
    r = nvfp4::launch_gemm_symmetric(pb, part, L.sym_bytes, s);
    if (r == NVFP4_EUNSUPPORTED) r = nvfp4::launch_gemm(pb, s);
    if (r != NVFP4_OK) return r;
    const float *clip_b = nullptr;
    if (cfg->clip_mask & 4u) {
      r = nvfp4::launch_abs_select(B, m, m, m, quantile_rank(cfg->clip_quantile, (uint64_t)(m * m)), sel(2), hist, compact, L.cap, s);
      if (r != NVFP4_OK) return r;
      clip_b = &sel(2)->value;
    }
    nvfp4::QuantProblem qb = make_quant(B, false, 1, m, m, m, m * m, false, &rne, &vB, base + L.ctrl[2]);
    qb.clip = clip_b;
    r = nvfp4::launch_quantize(qb, s);
    if (r != NVFP4_OK) return r;
    // X' = B X + a X, or its transpose X^T B^T + a X^T stored transposed
    // (the same products and sums, so the same values).
    nvfp4::GemmProblem px = make_gemm(&vB, &vXT, Xn, NVFP4_F32, ldn, m * ldn, 1.0f);
    if (transposed) {
      px = make_gemm(&vXT, &vB, Xn, NVFP4_F32, ldn, m * ldn, 1.0f);
      px.c_transposed = true;
    }
    px.cin = Xc;
    px.ldcin = ldc_;
    px.bstride_cin = m * ldc_;
    px.beta = ca;
    r = nvfp4::launch_gemm(px, s);
    if (r != NVFP4_OK) return r;
  }
  return NVFP4_OK;
}

// ---------------------------------------------------------------------------
// LoRA-style forward with the residual weight in NVFP4 and the low-rank
// subspace in BF16 ("Full-Stack FP4 ...", section 2.1).
// ---------------------------------------------------------------------------

namespace {

struct LoraLayout {
  size_t ctrl, codes, scales, st, t, total;
};

LoraLayout lora_layout(int64_t M, int64_t K, int64_t r) {
  LoraLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  L.ctrl = take(sizeof(QuantCtrl));
  L.codes = take((size_t)M * (size_t)K / 2);
  L.scales = take((size_t)M * (size_t)K / 16);
  L.st = take(sizeof(float));
  L.t = take((size_t)M * (size_t)r * 2);
  L.total = off;
  return L;
}

bool lora_shape_ok(int64_t M, int64_t K, int64_t r) {
  return M > 0 && K > 0 && K % 16 == 0 && r > 0 && r % 16 == 0 && r <= 128 && M <= kMaxExtent && K <= kMaxExtent;
}

}  // namespace

NVFP4_EXPORT size_t nvfp4_lora_workspace_size(int64_t M, int64_t K, int64_t r) {
  if (!lora_shape_ok(M, K, r)) return 0;
  return lora_layout(M, K, r).total;
}

NVFP4_EXPORT nvfp4_status nvfp4_lora_internals(void *workspace, size_t workspace_bytes, int64_t M, int64_t K,
                                               int64_t r, nvfp4_qtensor *x_view, uint16_t **t) {
  if (!workspace || !x_view || !t) return NVFP4_EINVAL;
  if (!lora_shape_ok(M, K, r)) return NVFP4_ESHAPE;
  const LoraLayout L = lora_layout(M, K, r);
  if (workspace_bytes < L.total) return NVFP4_EWORKSPACE;
  uint8_t *base = static_cast<uint8_t *>(workspace);
  x_view->codes = base + L.codes;
  x_view->scales = base + L.scales;
  x_view->tensor_scale = reinterpret_cast<float *>(base + L.st);
  x_view->batch = 1;
  x_view->rows = M;
  x_view->cols = K;
  *t = reinterpret_cast<uint16_t *>(base + L.t);
  return NVFP4_OK;
}

NVFP4_EXPORT nvfp4_status nvfp4_lora_forward(const void *x, const nvfp4_qtensor *w_res, const void *l1,
                                             const void *l2, int64_t M, int64_t N, int64_t K, int64_t r, float beta,
                                             void *y, int32_t y_dtype, int64_t ldy, void *workspace,
                                             size_t workspace_bytes, void *stream) {
  if (!x || !w_res || !l1 || !l2 || !y) return NVFP4_EINVAL;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (!(beta != 0.0f) || !std::isfinite(beta)) return NVFP4_EINVAL;
  if (!lora_shape_ok(M, K, r) || N <= 0 || N > kMaxExtent) return NVFP4_ESHAPE;
  nvfp4_status st = check_view(w_res, 1, N, K);
  if (st != NVFP4_OK) return st;
  if (ldy < N) return NVFP4_ESHAPE;
  if (!aligned(x, 16) || !aligned(l1, 16) || !aligned(l2, 16) || !aligned(y, y_dtype == NVFP4_F32 ? 4 : 2))
    return NVFP4_EALIGN;
  const LoraLayout L = lora_layout(M, K, r);
  if (!workspace || workspace_bytes < L.total) return NVFP4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_EALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  nvfp4_qtensor xv{};
  uint16_t *t = nullptr;
  nvfp4_lora_internals(workspace, workspace_bytes, M, K, r, &xv, &t);
  uint8_t *base = static_cast<uint8_t *>(workspace);
  const nvfp4_quant_opts rne{NVFP4_RNE, 0, 0, 0, 0u, 0u};
  st = nvfp4::launch_quantize(make_quant(x, true, 1, M, K, K, M * K, false, &rne, &xv, base + L.ctrl), s);
  if (st != NVFP4_OK) return st;
  st = nvfp4::launch_lora_down(static_cast<const uint16_t *>(x), M, K, K, static_cast<const uint16_t *>(l1), r, t, s);
  if (st != NVFP4_OK) return st;
  nvfp4::GemmProblem p = make_gemm(&xv, w_res, y, y_dtype, ldy, M * ldy, 1.0f);
  p.lr_t = t;
  p.lr_l2 = static_cast<const uint16_t *>(l2);
  p.lr_r = r;
  p.lr_beta = beta;
  return nvfp4::launch_gemm(p, s);
}
