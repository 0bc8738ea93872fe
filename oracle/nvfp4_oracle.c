/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for NVFP4 quantization and the
 * block-scaled GEMM that consumes it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The HIP library never
 * includes, links or calls anything in this directory, and this file shares no
 * header, table or helper with it.
 *
 * What the pages fix, and what this file therefore computes:
 *  - NVFP4 is a 4-bit floating-point element format used for the weights and
 *    activations that enter GEMMs, with BF16/FP32 kept for accumulators
 *    ("NVFP4 Treina com Precisao de 16 Bits...", TL;DR and FAQ;
 *    "NVIDIA acelera o pre-treinamento de LLM: NVFP4 no Blackwell...",
 *    section "Como o Treinamento Mixed-Precision Funciona com NVFP4").
 *  - The 4-bit grid is sparse, so it is paired with its own scaling scheme
 *    (same page, section "Por Que Cada Porcento E Importante").
 *  - Hadamard mixing spreads localised energy before quantization, and
 *    stochastic rounding is used on the gradient-like tensors
 *    ("Full-Stack FP4: Stable LLM Pretraining with Quantized Projections,
 *    Optimizers, and Attention", section 2.2).
 * The pages leave every numeric detail open.  The readings taken here are:
 *    elements: OCP MX E2M1 (values +-{0, .5, 1, 1.5, 2, 3, 4, 6});
 *    block scale: OCP FP8 E4M3FN, one per 16 contiguous contraction elements;
 *    tensor scale: FP32, s_t = amax / (6 * 448), stored as a decode factor;
 *    stochastic rounding driven by Philox4x32-10 (Salmon et al., SC'11);
 *    the Hadamard transform is the 16-point Sylvester matrix times a random
 *    +-1 diagonal, scaled by 1/4.
 * Steps are labelled Q0..Q9 (quantize) and G1..G2 (GEMM); each function says
 * which step it implements.  All FP32 arithmetic is IEEE binary32 with
 * round-to-nearest-even, no contraction into FMA (built with
 * -ffp-contract=off) and subnormals kept.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Bit helpers                                                               */
/* ------------------------------------------------------------------------ */

static float bits_to_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* BF16 is the upper half of a binary32, so widening is exact. */
static float bf16_to_float(uint16_t h) { return bits_to_float((uint32_t)h << 16); }

/* ------------------------------------------------------------------------ */
/* E2M1 (OCP MX FP4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.  */
/* ------------------------------------------------------------------------ */

/* Decode one 4-bit code to its value.  Exponent field 0 is subnormal. */
double oracle_e2m1_decode(int code) {
  int sign = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

/* Q8a: round-to-nearest-even onto the E2M1 grid with saturation at 6.
 * Each term counts one grid point passed; a tie goes to the neighbour whose
 * mantissa bit is 0, hence ">" at ties below an odd code and ">=" at ties
 * below an even code.  The sign bit is copied even when the magnitude
 * rounds to zero. */
int oracle_e2m1_encode_rne(float q) {
  float a = fabsf(q);
  int mag = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
            (a >= 3.5f) + (a > 5.0f);
  int sign = signbit(q) ? 1 : 0;
  return (sign << 3) | mag;
}

/* Q8b: stochastic rounding onto the E2M1 grid.  u is a uniform 16-bit word.
 * With lo the largest grid value <= a and delta the spacing above it, the
 * rounding fraction f = (a - lo) / delta (exact) is carried to 22 bits below
 * the E2M1 point, F = floor(f * 2^22), and the magnitude rounds up iff
 * 64 u < F, i.e. iff u / 2^16 < F / 2^22: with probability ceil(F / 64) /
 * 2^16.  (For a >= 1 F is exactly the 22 mantissa bits below the E2M1 one,
 * so there the rule is u / 2^16 < f.)  Saturates at 6. */
int oracle_e2m1_encode_sr(float q, uint32_t u) {
  static const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  float a = fminf(fabsf(q), 6.0f);
  int sign = signbit(q) ? 1 : 0;
  int mag;
  if (a == 6.0f) {
    mag = 7;
  } else {
    int lo_idx = 0;
    for (int i = 0; i < 7; ++i)
      if (grid[i] <= a) lo_idx = i;
    float delta = grid[lo_idx + 1] - grid[lo_idx];
    float f = (a - grid[lo_idx]) / delta;           /* exact: Sterbenz, power-of-two divisor */
    uint32_t F = (uint32_t)floorf(f * 4194304.0f);  /* exact scaling by 2^22, then the integer part */
    int up = (64u * (u & 0xFFFFu) < F) ? 1 : 0;
    mag = lo_idx + up;
  }
  return (sign << 3) | mag;
}

/* ------------------------------------------------------------------------ */
/* E4M3FN (OCP FP8): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,      */
/* no infinities, S.1111.111 is NaN, largest finite 448.                     */
/* ------------------------------------------------------------------------ */

double oracle_e4m3_decode(int byte) {
  int sign = (byte >> 7) & 1;
  int e = (byte >> 3) & 15;
  int m = byte & 7;
  double mag;
  if (e == 15 && m == 7)
    return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9); /* subnormal: m * 2^-6 / 8 */
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Q5 (encoding part): y >= 0 finite -> E4M3FN code, round-to-nearest-even,
 * values above 448 saturate to 448 (0x7E).  Subnormal and normal ranges are
 * handled separately; a mantissa that rounds up to 8 carries into the
 * exponent, which also turns the largest subnormal into 2^-6. */
int oracle_e4m3_encode_rne_sat(float y) {
  if (!(y > 0.0f))
    return 0;
  if (y > 448.0f)
    y = 448.0f;
  if (y < 0.015625f) { /* below 2^-6: subnormal step 2^-9 */
    double m = nearbyint((double)y * 512.0); /* exact scaling, RNE to integer */
    return (int)m; /* 0..8; 8 is the code of 2^-6 */
  }
  int e2;
  double fr = frexp((double)y, &e2); /* y = fr * 2^e2, fr in [0.5, 1) */
  int e = e2 - 1;                    /* y = (2 fr) * 2^e, 2 fr in [1, 2) */
  double m = nearbyint((2.0 * fr - 1.0) * 8.0);
  if (m == 8.0) {
    m = 0.0;
    e += 1;
  }
  return ((e + 7) << 3) | (int)m;
}

/* Array forms of the two encoders, for exhaustive sweeps in the tests. */
void oracle_e2m1_encode_rne_array(const float *q, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (uint8_t)oracle_e2m1_encode_rne(q[i]);
}

void oracle_e4m3_encode_rne_sat_array(const float *y, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (uint8_t)oracle_e4m3_encode_rne_sat(y[i]);
}

/* Stochastic rounding of value q[i] under word u[i], for i < n. */
void oracle_e2m1_encode_sr_pairs(const float *q, const uint32_t *u, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (uint8_t)oracle_e2m1_encode_sr(q[i], u[i]);
}

/* Stochastic rounding of each of nq values under every 16-bit word:
 * out[i * 65536 + u] = oracle_e2m1_encode_sr(q[i], u). */
void oracle_e2m1_encode_sr_all_words(const float *q, int64_t nq, uint8_t *out) {
  for (int64_t i = 0; i < nq; ++i)
    for (uint32_t u = 0; u < 65536u; ++u)
      out[i * 65536 + u] = (uint8_t)oracle_e2m1_encode_sr(q[i], u);
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As   */
/* Easy as 1, 2, 3", SC'11): 10 rounds of two 32x32->64 multiplies with an   */
/* S-box-free permutation; the key is bumped by two Weyl constants.          */
/* ------------------------------------------------------------------------ */

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t p0 = (uint64_t)M0 * c0;
    uint64_t p1 = (uint64_t)M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* Q8b: the random word for logical element n (row-major index in the
 * quantized view [batch][rows][cols]).  One Philox call serves 8 elements:
 * counter = (n/8 low, n/8 high, stream, 0), key = (seed low, seed high);
 * element n uses 16 bits of output word (n mod 8)/2, the low half for even n. */
uint32_t oracle_sr_word(uint64_t seed, uint32_t stream, uint64_t n) {
  uint64_t grp = n >> 3;
  uint32_t ctr[4] = {(uint32_t)grp, (uint32_t)(grp >> 32), stream, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  uint32_t w = out[(n & 7) >> 1];
  return (n & 1) ? (w >> 16) : (w & 0xFFFFu);
}

/* ------------------------------------------------------------------------ */
/* Q1: random Hadamard transform on a 16-element chunk.                      */
/* ------------------------------------------------------------------------ */

/* The +-1 diagonal: bit j of word 0 of Philox(counter=(0,0,~0,0),
 * key=seed) set means s_j = -1. */
void oracle_rht_signs(uint64_t seed, float s[16]) {
  uint32_t ctr[4] = {0u, 0u, 0xFFFFFFFFu, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  for (int j = 0; j < 16; ++j)
    s[j] = ((out[0] >> j) & 1u) ? -1.0f : 1.0f;
}

/* v <- (1/4) * H16 * diag(s) * v, with the Walsh-Hadamard butterflies taken
 * in the order h = 1, 2, 4, 8 in FP32 (H16 in Sylvester/natural order). */
void oracle_rht16(float v[16], const float s[16]) {
  float w[16];
  for (int j = 0; j < 16; ++j)
    w[j] = s[j] * v[j];
  for (int h = 1; h < 16; h <<= 1) {
    for (int i = 0; i < 16; ++i) {
      if (i & h)
        continue;
      float a = w[i], b = w[i + h];
      w[i] = a + b;
      w[i + h] = a - b;
    }
  }
  for (int j = 0; j < 16; ++j)
    v[j] = w[j] * 0.25f;
}

/* ------------------------------------------------------------------------ */
/* Q0..Q9: quantize one tensor.                                              */
/* ------------------------------------------------------------------------ */

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_ALONG_COLS = 0, ORACLE_ALONG_ROWS = 1 };
enum { ORACLE_RNE = 0, ORACLE_SR = 1 };

/* Q0: element (b, r, c) of the logical view.  For ALONG_COLS the logical
 * view is the input itself ([batch][rows][cols], row stride ld); for
 * ALONG_ROWS it is the transpose of each batch, so logical (b, r, c) is input
 * (b, c, r).  BF16 widens to FP32 exactly. */
static float load_logical(const void *x, int dtype, int axis, int64_t ld, int64_t bstride,
                          int64_t b, int64_t r, int64_t c) {
  int64_t row = (axis == ORACLE_ALONG_COLS) ? r : c;
  int64_t col = (axis == ORACLE_ALONG_COLS) ? c : r;
  int64_t off = b * bstride + row * ld + col;
  if (dtype == ORACLE_F32)
    return ((const float *)x)[off];
  return bf16_to_float(((const uint16_t *)x)[off]);
}

/* Quantize input x ([batch][in_rows][in_cols] with row stride ld and batch
 * stride bstride, in elements).  The quantized view has shape
 * [batch][qr][qc] with qc the contraction length (qc % 16 == 0):
 * ALONG_COLS: qr = in_rows, qc = in_cols;  ALONG_ROWS: qr = in_cols, qc = in_rows.
 * Outputs: codes [batch][qr][qc/2] (element 2j in the low nibble of byte j),
 * scales [batch][qr][qc/16] (E4M3 codes), *tensor_scale = s_t.
 * Returns 0, or -1 on a bad argument. */
int oracle_quantize(const void *x, int dtype, int64_t batch, int64_t in_rows, int64_t in_cols,
                    int64_t ld, int64_t bstride, int axis, int rounding, uint64_t sr_seed,
                    uint32_t sr_stream, int rht, uint64_t rht_seed, uint8_t *codes,
                    uint8_t *scales, float *tensor_scale) {
  int64_t qr = (axis == ORACLE_ALONG_COLS) ? in_rows : in_cols;
  int64_t qc = (axis == ORACLE_ALONG_COLS) ? in_cols : in_rows;
  if (batch < 0 || qr < 0 || qc < 0 || qc % 16 != 0)
    return -1;
  int64_t nblk = qc / 16;
  float signs[16];
  if (rht)
    oracle_rht_signs(rht_seed, signs);

  /* Q1 + Q2: transformed values are recomputed on each pass rather than
   * stored, so the oracle needs no buffer the size of the tensor. */
  float amax = 0.0f;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < qr; ++r)
      for (int64_t g = 0; g < nblk; ++g) {
        float v[16];
        for (int j = 0; j < 16; ++j)
          v[j] = load_logical(x, dtype, axis, ld, bstride, b, r, 16 * g + j);
        if (rht)
          oracle_rht16(v, signs);
        for (int j = 0; j < 16; ++j) {
          float a = fabsf(v[j]);
          if (isnan(a) || a > amax) /* a NaN input poisons s_t */
            amax = a;
        }
      }

  /* Q3, Q4 */
  float st = amax / 2688.0f;
  float d6 = 6.0f * st;
  *tensor_scale = st;

  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < qr; ++r)
      for (int64_t g = 0; g < nblk; ++g) {
        float v[16];
        for (int j = 0; j < 16; ++j)
          v[j] = load_logical(x, dtype, axis, ld, bstride, b, r, 16 * g + j);
        if (rht)
          oracle_rht16(v, signs);
        /* Q5: block scale */
        float ab = 0.0f;
        for (int j = 0; j < 16; ++j)
          ab = fmaxf(ab, fabsf(v[j]));
        int sbyte = 0;
        if (st > 0.0f) {
          float sb = ab / d6;
          sbyte = oracle_e4m3_encode_rne_sat(fminf(sb, 448.0f));
        }
        /* Q6: encode multiplier */
        float eb = (float)oracle_e4m3_decode(sbyte) * st;
        float rb = (eb == 0.0f) ? 0.0f : 1.0f / eb;
        /* Q7, Q8, Q9 */
        int64_t row_index = b * qr + r;
        for (int j = 0; j < 16; ++j) {
          float q = v[j] * rb;
          int code;
          if (rounding == ORACLE_SR) {
            uint64_t n = (uint64_t)(row_index * qc + 16 * g + j);
            code = oracle_e2m1_encode_sr(q, oracle_sr_word(sr_seed, sr_stream, n));
          } else {
            code = oracle_e2m1_encode_rne(q);
          }
          uint8_t *byte = &codes[row_index * (qc / 2) + 8 * g + j / 2];
          if (j % 2 == 0)
            *byte = (uint8_t)code;
          else
            *byte = (uint8_t)(*byte | (code << 4));
        }
        scales[row_index * nblk + g] = (uint8_t)sbyte;
      }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* G1: dequantize; G2: reference GEMM and its error bound.                   */
/* ------------------------------------------------------------------------ */

/* G1: value of element (row, k) of a quantized view with nk contraction
 * elements per row: E2M1(code) * E4M3(scale), exact in double.  The tensor
 * scale is not applied. */
static double deq(const uint8_t *codes, const uint8_t *scales, int64_t nk, int64_t row, int64_t k) {
  uint8_t byte = codes[row * (nk / 2) + k / 2];
  int code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
  return oracle_e2m1_decode(code) * oracle_e4m3_decode(scales[row * (nk / 16) + k / 16]);
}

/* Dequantize rows [0, rows) of one view (tensor scale applied) into out. */
void oracle_dequantize(const uint8_t *codes, const uint8_t *scales, float tensor_scale,
                       int64_t rows, int64_t nk, double *out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < nk; ++k)
      out[r * nk + k] = deq(codes, scales, nk, r, k) * (double)tensor_scale;
}

/* G2: for batch b and each selected row i of A, every column j:
 *   y_ref[i][j] = alpha * sA * sB * sum_k A^[b][i][k] * B^[b][j][k]
 *   sabs[i][j]  = |alpha| * sA * sB * sum_k |A^[b][i][k] * B^[b][j][k]|
 * in double.  A is [batch][M][K], B is [batch][N][K] (both quantized along
 * K).  rows == NULL selects all M rows; outputs are [nsel][N]. */
int oracle_gemm_ref(const uint8_t *a_codes, const uint8_t *a_scales, float a_st,
                    const uint8_t *b_codes, const uint8_t *b_scales, float b_st, int64_t M,
                    int64_t N, int64_t K, int64_t b, double alpha, const int64_t *rows,
                    int64_t nsel, double *y_ref, double *sabs) {
  if (K % 16 != 0)
    return -1;
  const uint8_t *ac = a_codes + b * M * (K / 2);
  const uint8_t *as = a_scales + b * M * (K / 16);
  const uint8_t *bc = b_codes + b * N * (K / 2);
  const uint8_t *bs = b_scales + b * N * (K / 16);
  double *bdeq = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  if (!bdeq || !arow) {
    free(bdeq);
    free(arow);
    return -2;
  }
  for (int64_t j = 0; j < N; ++j)
    for (int64_t k = 0; k < K; ++k)
      bdeq[j * K + k] = deq(bc, bs, K, j, k);
  double scale = alpha * (double)a_st * (double)b_st;
  int64_t count = rows ? nsel : M;
  for (int64_t t = 0; t < count; ++t) {
    int64_t i = rows ? rows[t] : t;
    for (int64_t k = 0; k < K; ++k)
      arow[k] = deq(ac, as, K, i, k);
    for (int64_t j = 0; j < N; ++j) {
      double s = 0.0, sa = 0.0;
      const double *brow = bdeq + j * K;
      for (int64_t k = 0; k < K; ++k) {
        double p = arow[k] * brow[k];
        s += p;
        sa += fabs(p);
      }
      y_ref[t * N + j] = scale * s;
      sabs[t * N + j] = fabs(scale) * sa;
    }
  }
  free(bdeq);
  free(arow);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* S1..S4: the AdamW moments held in NVFP4 ("Full-Stack FP4 ...", section    */
/* 2.2, Q-AdamW).  The page sends the first moment through the Hadamard     */
/* transform and stochastic rounding, and the second through a square root, */
/* a BF16 mean per tile taken out, the transform and NVFP4; reconstruction  */
/* undoes each step and squares.  Readings: the tile is the 16-element      */
/* NVFP4 block; the second moment rounds to nearest even; "adaptive 4/6     */
/* bit" is read as plain NVFP4.                                             */
/* ------------------------------------------------------------------------ */

/* RNE of a finite binary32 to BF16 bits (the upper half of the binary32 whose
 * value is nearest, ties to an even BF16 mantissa). */
static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lower = u & 0xFFFFu, upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
    upper += 1u;
  return (uint16_t)upper;
}

/* S1: one block of the second moment: s_j = sqrt(v_j) (IEEE, correctly
 * rounded), mu = BF16_RNE(fl(s_0 + ... + s_15) / 16) with the sum taken from
 * left to right, and the residuals r_j = fl(s_j - mu), returned in v.
 * Returns mu's BF16 bits. */
uint16_t oracle_sqrt_demean16(float v[16]) {
  float s[16];
  for (int j = 0; j < 16; ++j)
    s[j] = sqrtf(v[j]);
  float sum = s[0];
  for (int j = 1; j < 16; ++j)
    sum = sum + s[j];
  uint16_t mb = bf16_rne(sum / 16.0f);
  float mu = bf16_to_float(mb);
  for (int j = 0; j < 16; ++j)
    v[j] = s[j] - mu;
  return mb;
}

/* S2: encode m and v ([rows][cols] FP32, row stride ld, cols % 16 == 0).
 * m: the transform with rht_seed, then stochastic rounding with
 * (sr_seed, sr_stream), through oracle_quantize.  v: S1 on every block, then
 * the residuals through oracle_quantize with the transform and RNE.  Views
 * are [rows][cols] along cols; means are [rows][cols/16].  Returns 0, -1 on
 * a bad argument, -2 when out of memory. */
int oracle_qadamw_encode(const float *m, const float *v, int64_t rows, int64_t cols, int64_t ld,
                         uint64_t rht_seed, uint64_t sr_seed, uint32_t sr_stream,
                         uint8_t *m_codes, uint8_t *m_scales, float *m_st,
                         uint8_t *v_codes, uint8_t *v_scales, float *v_st, uint16_t *v_means) {
  if (rows < 0 || cols < 0 || cols % 16 != 0 || ld < cols)
    return -1;
  int rc = oracle_quantize(m, ORACLE_F32, 1, rows, cols, ld, rows * ld, ORACLE_ALONG_COLS,
                           ORACLE_SR, sr_seed, sr_stream, 1, rht_seed, m_codes, m_scales, m_st);
  if (rc != 0)
    return rc;
  float *res = (float *)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
  if (!res)
    return -2;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < cols / 16; ++g) {
      float b[16];
      for (int j = 0; j < 16; ++j)
        b[j] = v[r * ld + 16 * g + j];
      v_means[r * (cols / 16) + g] = oracle_sqrt_demean16(b);
      for (int j = 0; j < 16; ++j)
        res[r * cols + 16 * g + j] = b[j];
    }
  rc = oracle_quantize(res, ORACLE_F32, 1, rows, cols, cols, rows * cols, ORACLE_ALONG_COLS,
                       ORACLE_RNE, 0, 0, 1, rht_seed, v_codes, v_scales, v_st);
  free(res);
  return rc;
}

/* S3: the inverse transform of one dequantized block, the transform being
 * y = (1/4) H diag(s) x with H the 16-point Sylvester matrix (H H = 16 I):
 * x_j = s_j * (1/4) * sum_k H[j][k] * y_k, with y_k = E2M1 * E4M3 * s_t.
 * Every product and partial sum is exact in double (the y_k share the
 * factor E4M3 * s_t, and the sums of E2M1 values are small multiples of
 * 1/2), so the one rounding is the final conversion to FP32.  A sum that
 * is zero is +0 (the sum starts from +0), so a zero result takes the sign
 * of s_j.  H[j][k] = (-1)^popcount(j & k). */
static void inverse_transform_block(const uint8_t *codes, uint8_t scale, float st, const float s[16],
                                    float out[16]) {
  double y[16];
  for (int k = 0; k < 16; ++k) {
    int code = (k % 2 == 0) ? (codes[k / 2] & 0xF) : (codes[k / 2] >> 4);
    y[k] = oracle_e2m1_decode(code) * oracle_e4m3_decode(scale) * (double)st;
  }
  for (int j = 0; j < 16; ++j) {
    double acc = 0.0;
    for (int k = 0; k < 16; ++k)
      acc += (__builtin_popcount((unsigned)(j & k)) & 1) ? -y[k] : y[k];
    out[j] = (float)((double)s[j] * 0.25 * acc);
  }
}

/* S4: reconstruct m and v ([rows][cols], row stride ld) from the encoded
 * state: m_j = x_j; v_j = fl(fl(x_j + mu)^2) with mu the block's BF16
 * mean widened to FP32. */
int oracle_qadamw_decode(const uint8_t *m_codes, const uint8_t *m_scales, float m_st,
                         const uint8_t *v_codes, const uint8_t *v_scales, float v_st,
                         const uint16_t *v_means, int64_t rows, int64_t cols, int64_t ld,
                         uint64_t rht_seed, float *m, float *v) {
  if (rows < 0 || cols < 0 || cols % 16 != 0 || ld < cols)
    return -1;
  float signs[16];
  oracle_rht_signs(rht_seed, signs);
  int64_t nb = cols / 16;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < nb; ++g) {
      float x[16];
      inverse_transform_block(m_codes + r * (cols / 2) + 8 * g, m_scales[r * nb + g], m_st, signs, x);
      for (int j = 0; j < 16; ++j)
        m[r * ld + 16 * g + j] = x[j];
      inverse_transform_block(v_codes + r * (cols / 2) + 8 * g, v_scales[r * nb + g], v_st, signs, x);
      float mu = bf16_to_float(v_means[r * nb + g]);
      for (int j = 0; j < 16; ++j) {
        float sj = x[j] + mu;
        v[r * ld + 16 * g + j] = sj * sj;
      }
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* R1..R3: the pieces of Newton-Schulz in NVFP4 ("Full-Stack FP4 ...",       */
/* section 2.3, Q-Root) that are not a quantize or a GEMM.  Readings: the   */
/* p99 clip is the nearest-rank order statistic of |x| (the ceil(q N)-th    */
/* smallest), the tensor is clamped to [-p, p] before it is quantized, and  */
/* the iteration starts from G / (||G||_F + 1e-7).                          */
/* ------------------------------------------------------------------------ */

/* |x| as its bit pattern: for x >= 0 the patterns order like the values, and
 * NaN patterns sort above +inf. */
static uint32_t abs_key(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u & 0x7FFFFFFFu;
}

static int cmp_u32(const void *a, const void *b) {
  uint32_t x = *(const uint32_t *)a, y = *(const uint32_t *)b;
  return (x > y) - (x < y);
}

/* R1: the ceil(q n)-th smallest |x| (1-based, clamped to [1, n]) over x[0..n).
 * Returns 0, or -1 on a bad argument, -2 when out of memory. */
int oracle_abs_quantile(const float *x, int64_t n, double q, float *out) {
  if (n <= 0 || !(q > 0.0 && q <= 1.0))
    return -1;
  uint32_t *k = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)n);
  if (!k)
    return -2;
  for (int64_t i = 0; i < n; ++i)
    k[i] = abs_key(x[i]);
  qsort(k, (size_t)n, sizeof(uint32_t), cmp_u32);
  double r = ceil(q * (double)n);
  if (r < 1.0)
    r = 1.0;
  if (r > (double)n)
    r = (double)n;
  uint32_t v = k[(int64_t)r - 1];
  free(k);
  memcpy(out, &v, 4);
  return 0;
}

/* R2: out = x clamped to [-p, p] (NaN stays NaN). */
void oracle_clip(const float *x, int64_t n, float p, float *out) {
  for (int64_t i = 0; i < n; ++i) {
    float v = x[i];
    out[i] = (v > p) ? p : ((v < -p) ? -p : v);
  }
}

/* R3: the normalization factor fl32(1 / (||g||_F + 1e-7)), the sum of
 * squares taken in double, and x = fl(g * factor) ([rows][cols], g with row
 * stride ld, x contiguous). */
float oracle_frobenius_normalize(const void *g, int dtype, int64_t rows, int64_t cols, int64_t ld, float *x) {
  double s = 0.0;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      float v = load_logical(g, dtype, ORACLE_ALONG_COLS, ld, 0, 0, r, c);
      s += (double)v * (double)v;
    }
  float inv = (float)(1.0 / (sqrt(s) + 1e-7));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      x[r * cols + c] = load_logical(g, dtype, ORACLE_ALONG_COLS, ld, 0, 0, r, c) * inv;
  return inv;
}
