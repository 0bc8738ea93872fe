/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 quantize + block-scaled GEMM
 * library (libnvfp4.so).
 *
 * Pages cited below, by title:
 *   [P1] "NVFP4 Treina com Precisao de 16 Bits e a Velocidade de 4 Bits para
 *        Pre-treinamento em Grande Escala"
 *   [P2] "NVIDIA acelera o pre-treinamento de LLM: NVFP4 no Blackwell em
 *        conjunto com JAX e MaxText"
 *   [P3] "Full-Stack FP4: Stable LLM Pretraining with Quantized Projections,
 *        Optimizers, and Attention"
 *
 * What the library computes.  NVFP4 is a 4-bit floating-point format for the
 * weights and activations that enter the GEMMs of LLM training, with BF16 or
 * FP32 kept for the accumulators ([P2] "Como o Treinamento Mixed-Precision
 * Funciona com NVFP4"); the 4-bit grid is sparse, so it comes with its own
 * scaling scheme ([P2] "Por Que Cada Porcento E Importante").  Hadamard
 * mixing before quantization and stochastic rounding come from [P3] section
 * 2.2.  The pages leave the encoding open; the one used here:
 *   - element: OCP MX E2M1 (values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}), two codes
 *     per byte, element 2j in the low nibble of byte j;
 *   - block scale: OCP FP8 E4M3FN, one per 16 consecutive elements along the
 *     contraction (GEMM K) dimension;
 *   - tensor scale: FP32 s_t = fl(amax / 2688) with 2688 = 6 * 448, a decode
 *     factor (value = E2M1 * E4M3 * s_t).
 * Quantize steps, in order, for each 16-element block v of the logical view:
 *   (optional) v <- (1/4) H16 diag(s) v, FP32 butterflies in stage order 1,2,4,8;
 *   A = max |v| over the tensor;  s_t = fl(A / 2688);  D6 = fl(6 s_t);
 *   S = E4M3_RNE(min(fl(max|v in block| / D6), 448))  (S = 0 when s_t = 0);
 *   e = fl(E4M3(S) * s_t);  r = e ? fl(1 / e) : 0;  q = fl(v * r);
 *   code = E2M1 round-to-nearest-even(q) saturating at 6, or stochastic
 *   rounding with a 16-bit word from Philox4x32-10.
 *
 * Conventions for every entry point:
 *   - Pointers named in a struct or argument as "device" are device memory of
 *     the current HIP device; the structs themselves are host memory read
 *     during the call only.  The caller owns every buffer.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call except
 *     nvfp4_quantize_workspace_check only enqueues work on `stream`; none
 *     allocates.
 *   - Synchronous return codes report argument errors (checked before any HIP
 *     call) and launch failures.  Inputs must be finite and the tensor amax
 *     either 0 or >= 2^-100; a non-finite input leaves a non-finite tensor
 *     scale and unspecified codes.
 *   - Workspaces must be zero-filled before their first use.  Each call
 *     leaves the workspace ready for the next one (every counter a call uses
 *     is restored to zero by that call, whatever the grid size of the calls
 *     before or after it), so a workspace can be reused by later calls on the
 *     same stream without clearing.  Calls in flight at the same time need
 *     separate workspaces.  After NVFP4_EHIP or a barrier time-out (below),
 *     zero the workspace again.
 *   - Single-pass quantize launches (one workgroup per CU) meet at a
 *     grid-wide barrier for the tensor amax, so they need every CU to become
 *     free while they run.  The wait is bounded (about a second): if other
 *     work holds CUs for longer, the call's tensor scale is written as NaN
 *     (so every GEMM output that uses it is NaN) and the 32-bit time-out
 *     word at byte offset 8 of the control block becomes nonzero.  The word
 *     stays set, and every later single-pass call on that workspace also
 *     writes a NaN tensor scale, until the caller zeroes the workspace;
 *     nvfp4_quantize_workspace_check reports it.  The 32-bit word at byte
 *     offset 0 of a control block, if nonzero, replaces the default poll
 *     limit of that wait (for tests that force the time-out).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_EINVAL = 1,      /* null pointer, unknown enum value, inconsistent views */
  NVFP4_ESHAPE = 2,      /* contraction length not a multiple of 16, negative or oversized extents */
  NVFP4_EALIGN = 3,      /* a pointer or stride breaks the alignment stated below */
  NVFP4_EUNSUPPORTED = 4,/* a valid request the library does not implement */
  NVFP4_EHIP = 5,        /* the HIP runtime refused a launch or a copy */
  NVFP4_EWORKSPACE = 6,  /* workspace missing or smaller than the *_workspace_size() figure */
  NVFP4_ETIMEOUT = 7     /* a single-pass barrier wait on this workspace expired (results unreliable) */
} nvfp4_status;

typedef enum nvfp4_dtype { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;
typedef enum nvfp4_rounding { NVFP4_RNE = 0, NVFP4_SR = 1 } nvfp4_rounding;
/* ALONG_COLS: blocks run along the input's contiguous dimension; the
 * quantized view has the input's shape.  ALONG_ROWS: blocks run down the
 * input's columns; the quantized view is the per-batch transpose. */
typedef enum nvfp4_axis { NVFP4_ALONG_COLS = 0, NVFP4_ALONG_ROWS = 1 } nvfp4_axis;

/* One quantized view [batch][rows][cols], cols = contraction length (a
 * multiple of 16): the 4-bit weights or activations of [P2] "Como o
 * Treinamento Mixed-Precision Funciona com NVFP4" with their scaling scheme
 * ([P2] "Por Que Cada Porcento E Importante").  All three arrays are dense
 * and owned by the caller:
 *   codes        device, batch*rows*cols/2 bytes, 16-byte aligned;
 *   scales       device, batch*rows*cols/16 bytes (E4M3FN bit patterns,
 *                row-major, no swizzle), 4-byte aligned;
 *   tensor_scale device, one float (s_t), 4-byte aligned; written by the
 *                quantizer and read by the GEMM on the device (never copied
 *                to the host). */
typedef struct nvfp4_qtensor {
  uint8_t *codes;
  uint8_t *scales;
  float *tensor_scale;
  int64_t batch;
  int64_t rows;
  int64_t cols;
} nvfp4_qtensor;

/* Quantizer options ([P3] section 2.2: Hadamard mixing before quantization,
 * stochastic rounding).  rounding: an nvfp4_rounding.  rht: 0/1, apply the
 * 16-point random Hadamard transform along the contraction dimension first;
 * its +-1 diagonal is bit j of word 0 of Philox4x32-10(counter = (0, 0,
 * 0xFFFFFFFF, 0), key = rht_seed).  Stochastic rounding of logical element n
 * (row-major index in the quantized view) uses 16 bits of Philox4x32-10(
 * counter = (n/8 low, n/8 high, sr_stream, 0), key = sr_seed): the low half
 * of output word (n%8)/2 for even n, the high half for odd n; the magnitude
 * rounds up iff word < 2^16 * (|q| - lo) / (hi - lo). */
typedef struct nvfp4_quant_opts {
  int32_t rounding;
  int32_t rht;
  uint64_t sr_seed;
  uint64_t rht_seed;
  uint32_t sr_stream;
  uint32_t reserved; /* must be 0 */
} nvfp4_quant_opts;

/* Human-readable name of a status code (static storage). */
const char *nvfp4_status_string(int32_t status);

/* Library ABI version, (major << 16) | minor. */
int32_t nvfp4_version(void);

/* Bytes of workspace nvfp4_quantize needs (one 4 KiB control block). */
size_t nvfp4_quantize_workspace_size(void);

/* Quantize x to NVFP4: the per-tensor / per-block scaling of [P2] "Por Que
 * Cada Porcento E Importante" applied to a weight, activation or gradient
 * that enters a GEMM ([P2] "Como o Treinamento Mixed-Precision Funciona com
 * NVFP4"), with the options of [P3] section 2.2.
 *   x            device, [batch][rows][cols] elements of x_dtype with row
 *                stride ld >= cols and batch stride batch_stride >= rows*ld
 *                (elements).  ALONG_COLS: x, ld*esize and batch_stride*esize
 *                must be multiples of 16 bytes.  ALONG_ROWS: x must be aligned
 *                to its element size (16-byte aligned rows take the fast
 *                vector-load path).
 *   axis         ALONG_COLS: out has rows x cols, cols % 16 == 0.
 *                ALONG_ROWS: out has cols x rows (transpose), rows % 16 == 0.
 *   opts         host, may be NULL for RNE without transform.
 *   out          host struct describing the destination view; its batch, rows
 *                and cols must equal the view's shape.
 *   workspace    device, >= nvfp4_quantize_workspace_size() bytes, zeroed
 *                before first use, 256-byte aligned.
 * One tensor scale covers the whole view, all batches included (also for
 * batched attention operands).  Empty tensors (batch, rows or cols = 0) are
 * valid: nothing is written except tensor_scale = 0. */
nvfp4_status nvfp4_quantize(const void *x, int32_t x_dtype, int64_t batch, int64_t rows,
                            int64_t cols, int64_t ld, int64_t batch_stride, int32_t axis,
                            const nvfp4_quant_opts *opts, const nvfp4_qtensor *out,
                            void *workspace, size_t workspace_bytes, void *stream);

/* nvfp4_quantize without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments (minus the
 * workspace), checks and results, bit for bit.  Its scratch is one 4 KiB
 * control block, a static array of the library: one copy per GPU, zero
 * when the library's code is loaded, held until the process ends, looked up
 * once per device on that device's first call.  The call itself allocates
 * nothing.  Every quantize needs exactly one control block whatever its
 * size, so no size is refused for lack of scratch.  All calls of this entry
 * point on one GPU within a process share the block: calls that overlap in
 * time on one GPU (on different streams) race and give unspecified results,
 * so serialise them, or use nvfp4_quantize with separate workspaces.  A
 * barrier time-out (see the conventions) leaves the block's time-out word
 * set, after which every call of this entry point on that GPU publishes NaN
 * tensor scales for the rest of the process. */
nvfp4_status nvfp4_quantize_noalloc(const void *x, int32_t x_dtype, int64_t batch, int64_t rows,
                                    int64_t cols, int64_t ld, int64_t batch_stride, int32_t axis,
                                    const nvfp4_quant_opts *opts, const nvfp4_qtensor *out, void *stream);

/* Quantize one input in both orientations from one read: row_out as
 * nvfp4_quantize with ALONG_COLS ([batch][rows][cols]) and col_out as with
 * ALONG_ROWS ([batch][cols][rows]), each bit-identical to that call with its
 * own options (rounding, sr_seed, sr_stream), and one tensor scale, the same
 * in both views (without the transform both have the same maximum).  This is
 * how one tensor serves two GEMMs that contract over different dimensions:
 * [P3] section 2.4 quantizes Q, K and V once and reuses the quantized views
 * in the forward and the backward pass (QK^T contracts over the head
 * dimension, dS K and dS^T Q over the sequence).  rows % 16 == 0 and
 * cols % 16 == 0; x aligned to its element size (16-byte aligned rows take
 * the vector-load path); opts->rht must be 0 (NVFP4_EUNSUPPORTED otherwise);
 * opts may be NULL (RNE); workspace as for nvfp4_quantize.  Runs as two
 * passes over the input (tensor maximum, then both encodes). */
nvfp4_status nvfp4_quantize_dual(const void *x, int32_t x_dtype, int64_t batch, int64_t rows, int64_t cols,
                                 int64_t ld, int64_t batch_stride, const nvfp4_quant_opts *row_opts,
                                 const nvfp4_qtensor *row_out, const nvfp4_quant_opts *col_opts,
                                 const nvfp4_qtensor *col_out, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* One tensor of nvfp4_quantize_group: x as for nvfp4_quantize (ALONG_COLS). */
typedef struct nvfp4_quant_job {
  const void *x;
  int64_t batch, rows, cols, ld, batch_stride;
  nvfp4_qtensor out;
} nvfp4_quant_job;

/* Bytes of workspace nvfp4_quantize_group needs (16 KiB). */
size_t nvfp4_quantize_group_workspace_size(void);

/* Quantize the operands of one GEMM -- the weights and activations of [P2]
 * "Como o Treinamento Mixed-Precision Funciona com NVFP4" -- together: 1..4
 * tensors along their contiguous dimension with the same input dtype and
 * options, each with its own tensor scale.  The result equals
 * nvfp4_quantize on every job in turn (axis ALONG_COLS, same opts), bit for
 * bit.  Contiguous inputs (ld == cols, dense batches) whose blocks fit the
 * single-pass capacity together (on 256 CUs 37.7M BF16 elements, 29.4M
 * with both the transform and stochastic rounding, 16.8M FP32) are
 * quantized in one launch that reads every input once; other groups run as
 * separate calls.  Each job is validated as for nvfp4_quantize.  The
 * workspace (>= nvfp4_quantize_group_workspace_size(), 256-byte aligned)
 * follows the same rules: zeroed before first use, left reusable by each
 * call, one per concurrently running call. */
nvfp4_status nvfp4_quantize_group(const nvfp4_quant_job *jobs, int32_t njobs, int32_t x_dtype,
                                  const nvfp4_quant_opts *opts, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Diagnostic, and the one call that synchronises: waits for `stream`, then
 * reads the time-out word(s) of a quantize workspace (the one control block
 * of a >= 4 KiB workspace, both of a >= 16 KiB group workspace).  Returns
 * NVFP4_OK, NVFP4_ETIMEOUT if a single-pass barrier wait on it expired since
 * it was last zeroed, or an argument / NVFP4_EHIP error. */
nvfp4_status nvfp4_quantize_workspace_check(const void *workspace, size_t workspace_bytes, void *stream);

/* Block-scaled GEMM of two NVFP4 operands with wide accumulation, the GEMM
 * of [P2] "Como o Treinamento Mixed-Precision Funciona com NVFP4" (NVFP4
 * weights and activations, BF16/FP32 accumulators) and of [P3] section 1
 * (linear projections); batched, it is the QK^T scores product that [P3]
 * section 2.4 runs in NVFP4.  Both operands are quantized along K ("NT"):
 *   C[b][i][j] = alpha * sA * sB * sum_k A^[b][i][k] * B^[b][j][k]
 * with A^ = E2M1 * E4M3 (exact), sA/sB the tensor scales read on the device.
 * Accumulation is FP32; the epilogue multiplies by fl(fl(sA*sB)*alpha) and
 * stores FP32, or BF16 rounded to nearest even.
 *   a, b         host structs: a is [batch][M][K], b is [batch][N][K]
 *                (batch <= 65535 when the output is not empty).
 *   c            device, c_dtype elements, row stride ldc >= N, batch stride
 *                batch_stride_c >= M*ldc (elements), aligned to the element.
 * Any M, N >= 0 and K a multiple of 16 (K = 0 gives zeros).  The kernel and
 * tile shape are chosen per problem; results agree with the exact product
 * to the FP32 accumulation-order tolerance whatever the tile. */
nvfp4_status nvfp4_gemm(const nvfp4_qtensor *a, const nvfp4_qtensor *b, void *c, int32_t c_dtype,
                        int64_t ldc, int64_t batch_stride_c, float alpha, void *stream);

/* nvfp4_gemm with a requested workgroup tile (tile_m x tile_n), for tuning
 * and tests; the same product as nvfp4_gemm ([P2] "Como o Treinamento
 * Mixed-Precision Funciona com NVFP4").  tile_m = tile_n = 0 is the automatic
 * choice.  Tiles: 512x192 and 256x384 (eight-wavefront kernel; only where
 * K % 128 == 0 and each operand's codes are under 2 GiB), 256x256, 256x192
 * and 256x128 (four-wavefront kernel).  A tile that is not in this list or
 * does not apply to the problem returns NVFP4_EUNSUPPORTED. */
nvfp4_status nvfp4_gemm_ex(const nvfp4_qtensor *a, const nvfp4_qtensor *b, void *c, int32_t c_dtype,
                           int64_t ldc, int64_t batch_stride_c, float alpha, int32_t tile_m,
                           int32_t tile_n, void *stream);

/* nvfp4_gemm plus a scaled FP32 addend, the form of every Newton-Schulz
 * product of [P3] section 2.3 (X <- a X + (b A + c A A^T) X, run in NVFP4):
 *   C[b][i][j] = fl(fl(acc * fl(fl(sA*sB)*alpha)) + fl(beta * C_in[b][i][j]))
 * then stored as c_dtype (BF16: rounded to nearest even).
 *   c_in  device FP32 [batch][M][N], row stride ldc_in >= N, batch stride
 *         batch_stride_c_in >= M*ldc_in, 4-byte aligned.  It may be the output
 *         itself only as the very same FP32 array (same pointer, ldc and
 *         batch stride); any other overlap is undefined.
 * Otherwise as nvfp4_gemm. */
nvfp4_status nvfp4_gemm_axpby(const nvfp4_qtensor *a, const nvfp4_qtensor *b, void *c, int32_t c_dtype,
                              int64_t ldc, int64_t batch_stride_c, float alpha, const float *c_in,
                              int64_t ldc_in, int64_t batch_stride_c_in, float beta, void *stream);

/* Linear-layer training step in NVFP4: the quantized linear projections of
 * [P3] sections 1 and 2.1 (forward and backward GEMMs in NVFP4), stochastic
 * rounding and Hadamard mixing of [P3] section 2.2 on the gradient-side
 * operands; all inputs BF16, row-major:
 *   Fprop  Y  = X W^T  : X [M][K] and W [N][K] along K, RNE.
 *   Dgrad  dX = dY W   : dY [M][N] along N with stochastic rounding
 *                        (stream 1); W^T along N (transposing), RNE.
 *   Wgrad  dW = dY^T X : dY^T and X^T along M (transposing), both after the
 *                        random Hadamard transform (one rht_seed), stochastic
 *                        rounding on dY^T (stream 2) and, when wgrad_sr_x is
 *                        nonzero, on X^T (stream 3; RNE otherwise).
 * Y [M][N] and dX [M][K] are BF16; dW [N][K] has dtype dw_dtype.
 * M, N, K must be multiples of 16; all pointers 16-byte aligned.  The six
 * quantized views stay in the workspace after the call (nvfp4_linear_view). */
typedef struct nvfp4_linear_cfg {
  uint64_t sr_seed;
  uint64_t rht_seed;
  int32_t wgrad_sr_x;
  int32_t dw_dtype;
} nvfp4_linear_cfg;

/* Bytes of workspace for nvfp4_linear_fwd_bwd: the six quantized views and
 * their control blocks (0 for invalid sizes).  Zero it before first use. */
size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K);

nvfp4_status nvfp4_linear_fwd_bwd(const void *x, const void *w, const void *dy, void *y,
                                  void *dx, void *dw, int64_t M, int64_t N, int64_t K,
                                  const nvfp4_linear_cfg *cfg, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Describe quantized view `which` of a linear workspace (host computation
 * only, no HIP call), so that the views the step made can be reused instead
 * of quantized again -- the reuse of quantized views between forward and
 * backward of [P3] section 2.4:
 *   0: X [M][K]   1: W [N][K]   2: dY [M][N] (SR, stream 1)   3: W^T [K][N]
 *   4: dY^T [N][M] (RHT + SR, stream 2)   5: X^T [K][M] (RHT, SR stream 3
 *   or RNE).  Contents are defined once an nvfp4_linear_fwd_bwd call on this
 *   workspace has run on its stream. */
nvfp4_status nvfp4_linear_view(void *workspace, size_t workspace_bytes, int64_t M, int64_t N,
                               int64_t K, int32_t which, nvfp4_qtensor *out);

/* Attention backward through dS in NVFP4: [P3] section 2.4 runs QK^T and
 * dS in NVFP4 (keeping P V, P^T dO and dO V^T in BF16) and reuses the
 * quantized views of Q, K and V between the forward and the backward pass.
 * Given dS (the gradient of the scores, [bh][sq][sk], dtype ds_dtype,
 * contiguous) and the sequence-major quantized views q_seq [bh][d][sq] and
 * k_seq [bh][d][sk] (made once, e.g. by nvfp4_quantize_dual in the forward
 * pass, whose other view serves QK^T), this computes
 *   dQ[b] = alpha * dS[b] K[b]    ([bh][sq][d], row-major)
 *   dK[b] = alpha * dS[b]^T Q[b]  ([bh][sk][d], row-major)
 * in dtype out_dtype: dS is quantized in both orientations from one read
 * (nvfp4_quantize_dual; along the keys with stream 4, along the queries with
 * stream 5, rounding cfg->ds_rounding, seed cfg->sr_seed), then two batched
 * GEMMs as nvfp4_gemm.  sq, sk, d multiples of 16, bh <= 65535; ds, dq, dk
 * 16-byte aligned; workspace >= nvfp4_attention_ds_workspace_size(bh, sq,
 * sk) bytes, 256-byte aligned, zeroed before first use.  After the call the
 * workspace holds the two dS views, in order: along the keys [bh][sq][sk],
 * then along the queries [bh][sk][sq], each as codes, scales and a 256-byte
 * tensor-scale slot, every region starting on a 256-byte boundary; then one
 * quantize control block. */
typedef struct nvfp4_attn_cfg {
  uint64_t sr_seed;
  int32_t ds_rounding; /* NVFP4_SR (the gradient reading) or NVFP4_RNE */
  int32_t reserved;    /* 0 */
} nvfp4_attn_cfg;

size_t nvfp4_attention_ds_workspace_size(int64_t bh, int64_t sq, int64_t sk);

nvfp4_status nvfp4_attention_ds_grads(const void *ds, int32_t ds_dtype, const nvfp4_qtensor *q_seq,
                                      const nvfp4_qtensor *k_seq, void *dq, void *dk, int32_t out_dtype,
                                      int64_t bh, int64_t sq, int64_t sk, int64_t d, float alpha,
                                      const nvfp4_attn_cfg *cfg, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* Optimizer state of AdamW stored in NVFP4 ([P3] section 2.2, Q-AdamW): the
 * first moment m is passed through the 16-point random Hadamard transform
 * and quantized with stochastic rounding; the second moment v (v >= 0) goes
 * through a square root, a block mean taken out and kept in BF16 (the "tile"
 * is the 16-element NVFP4 block: mu = BF16_RNE(fl(sum_j sqrt(v_j)) / 16),
 * summed left to right), and the transform of the residual sqrt(v_j) - mu,
 * quantized with round-to-nearest-even.  Reconstruction inverts each step in
 * FP32: x = fl(E2M1 * E4M3 * s_t), the inverse transform (1/4) D H, then for
 * the second moment fl(fl(x + mu)^2).  Both views are [1][rows][cols] along
 * cols; one tensor scale each; the same rht_seed for encode and decode. */
typedef struct nvfp4_qadamw_state {
  nvfp4_qtensor m;    /* first moment, transformed, stochastic rounding */
  nvfp4_qtensor v;    /* residual of sqrt(second moment) after its block means, transformed, RNE */
  uint16_t *v_means;  /* device, rows*cols/16 BF16 block means of sqrt(v), 2-byte aligned */
} nvfp4_qadamw_state;

/* Bytes of workspace nvfp4_qadamw_encode needs (two quantize control blocks). */
size_t nvfp4_qadamw_workspace_size(void);

/* Encode FP32 moments m, v ([rows][cols], row stride ld floats, 16-byte
 * aligned rows, cols % 16 == 0) into `state` (device arrays owned by the
 * caller).  Stochastic rounding of m uses sr_seed and stream sr_stream as in
 * nvfp4_quant_opts.  Workspace as for nvfp4_quantize (8 KiB, zeroed before
 * first use, reusable). */
nvfp4_status nvfp4_qadamw_encode(const float *m, const float *v, int64_t rows, int64_t cols, int64_t ld,
                                 uint64_t rht_seed, uint64_t sr_seed, uint32_t sr_stream,
                                 const nvfp4_qadamw_state *state, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Reconstruct FP32 moments m, v ([rows][cols] with row stride ld, 16-byte
 * aligned rows) from `state`. */
nvfp4_status nvfp4_qadamw_decode(const nvfp4_qadamw_state *state, uint64_t rht_seed, float *m, float *v, int64_t ld,
                                 void *stream);

/* Newton-Schulz orthogonalization with every matrix product in NVFP4, the
 * Q-Root recipe of [P3] section 2.3 (the products run directly in NVFP4,
 * stabilised by per-step coefficients a, b, c and clipping of p99 outliers):
 *   X_0 = G / (||G||_F + 1e-7)   (norm in FP64, factor rounded to FP32)
 *   for k = 0 .. steps-1, with (a, b, c) = coeffs[3k .. 3k+2]:
 *     X^  = NVFP4 of clip(X_k) along its rows, X^T^ = NVFP4 of clip(X_k)^T
 *     A   = X^ X^^T                          (FP32 [m][m])
 *     B   = c * A^ A^^T + b * A             (A^ = NVFP4 of clip(A); A is symmetric)
 *     X_{k+1} = B^ X^ + a * X_k             (B^ = NVFP4 of clip(B))
 * every GEMM through the block-scaled kernel with the FP32 addend epilogue
 * of nvfp4_gemm_axpby, every quantization RNE without the transform.
 * clip(T) clamps T to [-p, p] with p the clip_quantile order statistic of
 * |T| (the ceil(q * numel)-th smallest, exact), for the tensors selected by
 * clip_mask (bit 0: X, bit 1: A, bit 2: B); the FP32 terms a X_k and b A use
 * the unclipped tensors.  The page gives neither the coefficients nor the
 * tensors clipped: both are the caller's.
 *   g     device [m][n], dtype g_dtype, row stride ldg (multiple of 4),
 *         16-byte aligned (8 for BF16);  m, n multiples of 16, m*n < 4e9.
 *   coeffs  host, 3*steps floats; steps in [0, 64] (0: X = X_0).
 *   x     device FP32 [m][n] output, row stride ldx (multiple of 4), 16-byte
 *         aligned; it must not overlap g or the workspace.
 * The caller passes the orientation it wants orthogonalized (A is m x m:
 * m <= n is the cheap one).  Workspace: nvfp4_ns_workspace_size(m, n)
 * bytes, 256-byte aligned, zeroed before first use, reusable; after a call
 * it holds the last step's intermediates (nvfp4_ns_internals). */
typedef struct nvfp4_ns_cfg {
  double clip_quantile;  /* in (0, 1]; 0.99 is the page's p99 */
  uint32_t clip_mask;    /* bit 0: X, bit 1: A, bit 2: B; 0: no clipping */
  uint32_t product;      /* how B^ X^ is launched: 0 automatic, 1 as the [m][n]
                            product, 2 as its transpose X^T^ B^^T ([n][m], the
                            workgroup tiles of the [n][m] shape may fill the GPU
                            better) stored transposed.  The same products and
                            sums either way; 0 picks the one with fewer rounds
                            of workgroup tiles. */
} nvfp4_ns_cfg;

size_t nvfp4_ns_workspace_size(int64_t m, int64_t n);

nvfp4_status nvfp4_ns_orthogonalize(const void *g, int32_t g_dtype, int64_t m, int64_t n, int64_t ldg,
                                    const float *coeffs, int32_t steps, const nvfp4_ns_cfg *cfg, float *x,
                                    int64_t ldx, void *workspace, size_t workspace_bytes, void *stream);

/* Where the last step's intermediates live in a Newton-Schulz workspace
 * (host computation only): x_prev = X_{steps-1} ([m][n], row stride n; valid
 * when steps >= 1), a = A and b = B ([m][m] FP32), clip[i] = the clip value
 * of X, A, B (device floats; valid when that bit was set), inv_norm = the
 * normalization factor, and the quantized views 0: X^ [m][n], 1: X^T^
 * [n][m], 2: A^ [m][m], 3: B^ [m][m]. */
typedef struct nvfp4_ns_state {
  float *x_prev;
  float *a;
  float *b;
  const float *clip[3];
  const float *inv_norm;
  nvfp4_qtensor view[4];
} nvfp4_ns_state;

nvfp4_status nvfp4_ns_internals(void *workspace, size_t workspace_bytes, int64_t m, int64_t n,
                                nvfp4_ns_state *out);

/* Forward of a linear layer parametrized as W = W_res + beta L2 L1 ([P3]
 * section 2.1, LoRA-SVD: the dominant residual W_res in NVFP4, the compact
 * subspace L2 L1 kept in BF16):
 *   T = BF16_RNE(X L1^T)                 (FP32 accumulation)
 *   Y = s * X^ W_res^^T + beta * T L2^T   (FP32 accumulation, then y_dtype)
 * with X^ the NVFP4 view of X (RNE, no transform; stays in the workspace),
 * s = fl(fl(sX sW) * 1).  The low-rank product is folded into the NVFP4
 * GEMM's FP32 accumulators before its main loop, pre-divided by s (q =
 * fl(beta / s); q = 1 and factor beta when s = 0), so Y agrees with the
 * exact s * sum + beta * T L2^T to the FP32 accumulation tolerance; results
 * are unspecified if fl(beta / s) overflows.
 *   x      device BF16 [M][K], contiguous, 16-byte aligned.
 *   w_res  host struct, the NVFP4 view [1][N][K] of W_res.
 *   l1     device BF16 [r][K], l2 device BF16 [N][r], contiguous, 16-byte
 *          aligned; r a multiple of 16, 16 <= r <= 128.
 *   beta   finite and nonzero.
 *   y      device [M][N], dtype y_dtype, row stride ldy.
 * K a multiple of 16.  Workspace: nvfp4_lora_workspace_size(M, K, r) bytes,
 * 256-byte aligned, zeroed before first use; it keeps X^ and T. */
size_t nvfp4_lora_workspace_size(int64_t M, int64_t K, int64_t r);

nvfp4_status nvfp4_lora_forward(const void *x, const nvfp4_qtensor *w_res, const void *l1, const void *l2,
                                int64_t M, int64_t N, int64_t K, int64_t r, float beta, void *y, int32_t y_dtype,
                                int64_t ldy, void *workspace, size_t workspace_bytes, void *stream);

/* The view X^ ([1][M][K]) and T (device BF16 [M][r]) a LoRA workspace holds
 * (host computation only). */
nvfp4_status nvfp4_lora_internals(void *workspace, size_t workspace_bytes, int64_t M, int64_t K, int64_t r,
                                  nvfp4_qtensor *x_view, uint16_t **t);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
