/*
 * qlora_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU statement of what the QLoRA
 * frozen-base LoRA linear layer computes: NF4 blockwise quantization with
 * double quantization of the block scales, double dequantization to BF16,
 * and the LoRA linear forward and backward.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load this file's
 * library.  It shares no code, header, table or constant with the HIP
 * library; the two meet only at the seeded inputs that the tests hand to
 * both.
 *
 * Sources (the pages): "第 04 篇：QLoRA 原理" (jupiter-lab, QLoRA principles),
 * cited as [QP §x.y], and "QLoRA" (compassingai concept page, "NF4 量化機制詳解"
 * and "雙重量化"), cited as [CP, <heading>].
 *
 * Every floating-point decision that fixes an integer (an NF4 index, an FP8
 * code, a BF16 pattern) is taken by exact comparison of distances, not by
 * bit tricks, so that a reader can check each against its definition.
 * Matrix products accumulate in FP64 over exactly-represented inputs.
 *
 * Readings where the pages are silent:
 *   - flatten order is row-major over W[d_out, d_in]; blocks of 64 follow it;
 *   - x = w / absmax is an IEEE FP32 division; a zero block maps to index 7;
 *   - nearest-level ties go to the lower index;
 *   - element 2j is the low nibble of byte j;
 *   - the scale mean is one FP32 value per tensor, summed in FP64 by a fixed
 *     stride-halving tree (per 256-group, then over the groups);
 *   - "symmetric 8-bit" second-level quantization is OCP FP8 E4M3FN with the
 *     group's largest |centred scale| mapped to 448, round-to-nearest-even,
 *     saturating; an all-zero group stores code 0;
 *   - restored scale = fp8(code) * s2 + mean (FP32, two roundings, no FMA);
 *     restored weight = RNE_bf16(codebook[idx] * restored scale) (FP32 product);
 *   - LoRA dropout is inverted dropout on the LoRA branch's input, its mask
 *     drawn from Philox4x32-10 by element position (orc_dropout_keep).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BLOCK 64   /* first-level block size B1   [QP §3.4, §5.1] */
#define ORC_GROUP 256  /* second-level block size B2  [QP §5.2]; [CP, 雙重量化] */

/* ------------------------------------------------------------------------
 * NF4 codebook: the 16 values printed in [QP §4.3] (the bitsandbytes table
 * quoted there), parsed as FP32 by the C library.
 * ---------------------------------------------------------------------- */
static const char *const ORC_NF4_TEXT[16] = {
    "-1.0000000", "-0.6961928", "-0.5250731", "-0.3949175",
    "-0.2844414", "-0.1847734", "-0.0910500", "0.0000000",
    "0.0795803",  "0.1609302",  "0.2461123",  "0.3379152",
    "0.4407098",  "0.5626170",  "0.7229568",  "1.0000000"};

static float ORC_NF4[16];

__attribute__((constructor)) static void orc_parse_codebook(void) {
  for (int i = 0; i < 16; ++i) ORC_NF4[i] = strtof(ORC_NF4_TEXT[i], NULL);
}

void orc_codebook(float out[16]) {
  for (int i = 0; i < 16; ++i) out[i] = ORC_NF4[i];
}

/* Nearest NF4 level to x (x is a normalized weight in [-1, 1]):
 * argmin_i |x - c_i|, the first (lowest) index on a tie.  [CP, NF4 量化機制詳解
 * step 3: map the normalized value to the nearest NF4 level.]  The distances
 * are FP64 differences of two FP32 values; wherever two distances are close
 * enough to compete, x and the levels are of similar magnitude and the
 * differences are exact. */
uint8_t orc_nf4_index(float x) {
  const float *c = ORC_NF4;
  int best = 0;
  double bestd = fabs((double)x - (double)c[0]);
  for (int i = 1; i < 16; ++i) {
    double d = fabs((double)x - (double)c[i]);
    if (d < bestd) { bestd = d; best = i; }
  }
  return (uint8_t)best;
}

/* ------------------------------------------------------------------------
 * FP8 E4M3FN (OCP 8-bit floating point, "FN" = finite + NaN, no infinities):
 * sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0
 * holds subnormals m * 2^-9; S.1111.111 is NaN; the largest finite is 448.
 * ---------------------------------------------------------------------- */
float orc_fp8_decode(uint8_t code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) mag = ldexp((double)m, -9);
  else mag = ldexp(1.0 + m / 8.0, e - 7);
  return (float)(s ? -mag : mag);
}

/* The 127 non-negative finite E4M3FN magnitudes, code 0x00..0x7E, as
 * decoded above (filled once when the library loads). */
static double ORC_FP8_MAG[0x7F];

__attribute__((constructor)) static void orc_fp8_table(void) {
  for (int code = 0; code <= 0x7E; ++code) ORC_FP8_MAG[code] = (double)orc_fp8_decode((uint8_t)code);
}

/* Encode y as the nearest of the 127 non-negative finite E4M3FN magnitudes
 * (codes 0x00..0x7E, increasing), ties to the even code, |y| beyond 448
 * clamped to 448, sign bit = sign bit of y.  Never produces NaN. */
uint8_t orc_fp8_encode(float y) {
  double a = fabs((double)y);
  int best = 0x7E;                 /* |y| >= 448: the largest finite, 448 */
  double bestd = INFINITY;
  for (int code = 0; code <= 0x7E && a < 448.0; ++code) {
    double v = ORC_FP8_MAG[code];
    double d = fabs(a - v);
    if (d < bestd || (d == bestd && (code & 1) == 0 && (best & 1) == 1)) {
      bestd = d;
      best = code;
    }
  }
  return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* ------------------------------------------------------------------------
 * BF16: the upper 16 bits of an FP32 pattern.  Round-to-nearest-even is
 * written out as: the two BF16 neighbours of x (toward zero and away from
 * zero), the closer one wins, a tie goes to the even mantissa.
 * ---------------------------------------------------------------------- */
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float orc_bf16_to_float(uint16_t h) { return u2f((uint32_t)h << 16); }

static double bf16_pattern_value(uint32_t hi16) {
  /* magnitude of a non-negative BF16 pattern; the pattern just past the
   * largest finite value stands for 2^128 when measuring distances. */
  if ((hi16 & 0x7FFF) == 0x7F80) return ldexp(1.0, 128);
  return (double)orc_bf16_to_float((uint16_t)hi16);
}

uint16_t orc_bf16_rne(float x) {
  uint32_t u = f2u(x);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040);
  if (isinf(x)) return (uint16_t)(u >> 16);
  uint32_t sign = u & 0x80000000u, mag = u & 0x7FFFFFFFu;
  uint32_t lo = mag >> 16;      /* neighbour toward zero  */
  uint32_t hi = lo + 1;          /* neighbour away from zero */
  double ax = (double)u2f(mag);
  double dlo = ax - bf16_pattern_value(lo);
  double dhi = bf16_pattern_value(hi) - ax;
  uint32_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = (lo & 1) ? hi : lo;
  return (uint16_t)((sign >> 16) | pick);
}

/* ------------------------------------------------------------------------
 * Quantization [QP §3.4, §4.3, §5.2, §6.1]; [CP, NF4 量化機制詳解; 雙重量化]
 *
 * W is n = d_out*d_in FP32 values flattened row-major; n % 64 == 0.
 * Outputs: codes[n/2] (two 4-bit indices per byte, element 2j low nibble,
 * [QP §2.1]), scale_codes[n/64] (FP8 E4M3FN), s2[ceil(n1/256)] (FP32
 * second-level scales), *mean (FP32 offset subtracted before the second
 * level).  absmax_out (optional) receives the FP32 first-level absmax.
 * ---------------------------------------------------------------------- */

/* Stride-halving FP64 tree over v[0..len), len a power of two:
 * v[j] += v[j + half] for half = len/2, len/4, ..., 1.  Returns v[0]. */
static double tree_sum(double *v, int64_t len) {
  for (int64_t half = len / 2; half >= 1; half /= 2)
    for (int64_t j = 0; j < half; ++j) v[j] = v[j] + v[j + half];
  return v[0];
}

/* Mean of the n1 first-level scales, summed in groups of B2 (a power of
 * two) by the stride-halving tree, then by the same tree over the group
 * sums padded with zeros to a power of two; quotient rounded to FP32. */
float orc_scale_mean_g(const float *absmax, int64_t n1, int64_t B2) {
  int64_t G = (n1 + B2 - 1) / B2;
  int64_t Gp = 1;
  while (Gp < G) Gp *= 2;
  double *part = (double *)calloc((size_t)Gp, sizeof(double));
  double *grp = (double *)malloc((size_t)B2 * sizeof(double));
  for (int64_t g = 0; g < G; ++g) {
    for (int64_t j = 0; j < B2; ++j) {
      int64_t b = g * B2 + j;
      grp[j] = (b < n1) ? (double)absmax[b] : 0.0;
    }
    part[g] = tree_sum(grp, B2);
  }
  double S = tree_sum(part, Gp);
  free(grp);
  free(part);
  return (float)(S / (double)n1);
}

float orc_scale_mean(const float *absmax, int64_t n1) {
  return orc_scale_mean_g(absmax, n1, ORC_GROUP);
}

/* General block sizes [QP §5.5]: first-level blocks of B1 consecutive
 * elements, second-level groups of B2 consecutive block scales (both powers
 * of two), any n >= 1.  A last block shorter than B1 (n % B1 != 0) takes the
 * absmax of the elements it has; a last group shorter than B2 likewise.
 * codes has ceil(n/2) bytes; for odd n the high nibble of the last byte,
 * which no element owns, is 0.  B1 = 64, B2 = 256 and n % 64 == 0 is the
 * layer format above.
 * group_sel (NULL: every group) limits the NF4 codes to the blocks of the
 * groups g with group_sel[g] != 0; the codes of other blocks are left 0.
 * Absmax, mean, second-level scales and FP8 codes are always computed for
 * every block, since the mean depends on all of them. */
static void quantize_impl(const float *W, int64_t n, int64_t B1, int64_t B2,
                          const uint8_t *group_sel, uint8_t *codes, uint8_t *scale_codes,
                          float *s2, float *mean, float *absmax_out) {
  int64_t n1 = (n + B1 - 1) / B1;
  int64_t G = (n1 + B2 - 1) / B2;
  float *a = (float *)malloc((size_t)n1 * sizeof(float));
  memset(codes, 0, (size_t)((n + 1) / 2));

  /* First level: absmax per block, normalize, nearest level, pack. */
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < n1; ++b) {
    const int64_t e0 = b * B1;
    const int64_t len = (n - e0 < B1) ? n - e0 : B1;
    float m = 0.0f;
    for (int64_t j = 0; j < len; ++j) {
      float v = fabsf(W[e0 + j]);
      if (v > m) m = v;
    }
    a[b] = m;
    if (group_sel && !group_sel[b / B2]) continue;
    /* B1 is even, so a block owns whole bytes */
    for (int64_t j = 0; j < len; ++j) {
      float x = (m == 0.0f) ? 0.0f : W[e0 + j] / m;
      uint8_t idx = orc_nf4_index(x);
      int64_t e = e0 + j;
      codes[e / 2] = (uint8_t)(codes[e / 2] | (e % 2 == 0 ? idx : (uint8_t)(idx << 4)));
    }
  }
  if (absmax_out) memcpy(absmax_out, a, (size_t)n1 * sizeof(float));

  /* Second level: subtract the mean, then per group an FP32 scale
   * s2 = max|centred| / 448 and FP8 codes of centred / s2.  Groups are
   * independent of one another. */
  float mu = orc_scale_mean_g(a, n1, B2);
  *mean = mu;
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < G; ++g) {
    int64_t b0 = g * B2, b1 = b0 + B2;
    if (b1 > n1) b1 = n1;
    float mg = 0.0f;
    for (int64_t b = b0; b < b1; ++b) {
      float d = fabsf(a[b] - mu);
      if (d > mg) mg = d;
    }
    float sc = mg / 448.0f;
    s2[g] = sc;
    for (int64_t b = b0; b < b1; ++b) {
      float d = a[b] - mu;
      scale_codes[b] = (sc == 0.0f) ? (uint8_t)0 : orc_fp8_encode(d / sc);
    }
  }
  free(a);
}

void orc_quantize_nf4_blocked(const float *W, int64_t n, int64_t B1, int64_t B2,
                              uint8_t *codes, uint8_t *scale_codes, float *s2,
                              float *mean, float *absmax_out) {
  quantize_impl(W, n, B1, B2, NULL, codes, scale_codes, s2, mean, absmax_out);
}

void orc_quantize_nf4(const float *W, int64_t n, uint8_t *codes,
                      uint8_t *scale_codes, float *s2, float *mean,
                      float *absmax_out) {
  quantize_impl(W, n, ORC_BLOCK, ORC_GROUP, NULL, codes, scale_codes, s2, mean, absmax_out);
}

/* The layer format with NF4 codes only for the selected groups (see
 * quantize_impl); everything else as orc_quantize_nf4. */
void orc_quantize_nf4_sel(const float *W, int64_t n, const uint8_t *group_sel,
                          uint8_t *codes, uint8_t *scale_codes, float *s2, float *mean) {
  quantize_impl(W, n, ORC_BLOCK, ORC_GROUP, group_sel, codes, scale_codes, s2, mean, NULL);
}

/* Restored first-level scale of block b [QP §5.2 restore order; §6.1]. */
float orc_restored_scale_g(const uint8_t *scale_codes, const float *s2,
                           float mean, int64_t b, int64_t B2) {
  volatile float p = orc_fp8_decode(scale_codes[b]) * s2[b / B2];
  return p + mean;
}

float orc_restored_scale(const uint8_t *scale_codes, const float *s2,
                         float mean, int64_t b) {
  return orc_restored_scale_g(scale_codes, s2, mean, b, ORC_GROUP);
}

/* Double dequantization to BF16 [QP §2.3, §6.1]: restored weight of element
 * e is RNE_bf16(codebook[idx_e] * restored_scale(block of e)). */
void orc_dequant_bf16_blocked(const uint8_t *codes, const uint8_t *scale_codes,
                              const float *s2, float mean, int64_t n, int64_t B1,
                              int64_t B2, uint16_t *out) {
  float c[16];
  orc_codebook(c);
  int64_t n1 = (n + B1 - 1) / B1;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < n1; ++b) {
    float ah = orc_restored_scale_g(scale_codes, s2, mean, b, B2);
    for (int64_t j = 0; j < B1 && b * B1 + j < n; ++j) {
      int64_t e = b * B1 + j;
      uint8_t byte = codes[e / 2];
      int idx = (e % 2 == 0) ? (byte & 15) : (byte >> 4);
      volatile float prod = c[idx] * ah;
      out[e] = orc_bf16_rne(prod);
    }
  }
}

void orc_dequant_bf16(const uint8_t *codes, const uint8_t *scale_codes,
                      const float *s2, float mean, int64_t n, uint16_t *out) {
  orc_dequant_bf16_blocked(codes, scale_codes, s2, mean, n, ORC_BLOCK, ORC_GROUP, out);
}

/* ------------------------------------------------------------------------
 * LoRA linear, forward and backward [QP §1.2, §2.2, §2.4, §6.3, §6.4].
 * Column-vector statement y = W x + s B A x with s = alpha / r, written for
 * row-major token matrices: Y = X Wh^T + s (X A^T) B^T.
 *   Wh [d_out, d_in] restored weights, X [M, d_in], A [r, d_in], B [d_out, r].
 * Inputs are FP32 arrays holding the exact values (BF16 values in use);
 * every product and sum is FP64.  No gradient is formed for Wh.
 * ---------------------------------------------------------------------- */

/* LoRA dropout in training mode [QP §6.3]: the LoRA branch sees
 * D(x) = keep * x / (1 - p) instead of x; the base branch sees x.  keep is a
 * row-major [M, d_in] array of 0/1 (NULL: no dropout, D(x) = x) and
 * keep_prob = 1 - p.  The value is formed in FP64. */
static double lora_input(const float *X, const uint8_t *keep, double keep_prob,
                         int64_t idx) {
  if (!keep) return (double)X[idx];
  return keep[idx] ? (double)X[idx] / keep_prob : 0.0;
}

/* Y rows listed in rows[0..nrows): Y[k, :] for token rows[k]. */
void orc_linear_fwd_rows(const float *Wh, const float *X, const float *A,
                         const float *B, int64_t d_out, int64_t d_in,
                         int64_t r, double s, const int64_t *rows,
                         int64_t nrows, const uint8_t *keep, double keep_prob,
                         double *Y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < nrows; ++k) {
    const float *x = X + rows[k] * d_in;
    double *t = (double *)malloc((size_t)(r > 0 ? r : 1) * sizeof(double));
    for (int64_t i = 0; i < r; ++i) {          /* t = A D(x)     */
      double acc = 0.0;
      for (int64_t c = 0; c < d_in; ++c)
        acc += (double)A[i * d_in + c] * lora_input(X, keep, keep_prob, rows[k] * d_in + c);
      t[i] = acc;
    }
    for (int64_t o = 0; o < d_out; ++o) {      /* y = Wh x + s B t */
      double base = 0.0;
      for (int64_t c = 0; c < d_in; ++c) base += (double)Wh[o * d_in + c] * x[c];
      double lora = 0.0;
      for (int64_t i = 0; i < r; ++i) lora += (double)B[o * r + i] * t[i];
      Y[k * d_out + o] = base + s * lora;
    }
    free(t);
  }
}

/* The LoRA branch's rank-r intermediate alone [QP §2.2]:
 *   T[m, i] = s * sum over c ascending of A[i, c] D(X)[m, c]     [M, r]
 * (the quantity the forward hands to the backward).  FP64. */
void orc_lora_down(const float *X, const float *A, int64_t M, int64_t d_in, int64_t r,
                   double s, const uint8_t *keep, double keep_prob, double *T) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t i = 0; i < r; ++i) {
      double acc = 0.0;
      for (int64_t c = 0; c < d_in; ++c)
        acc += (double)A[i * d_in + c] * lora_input(X, keep, keep_prob, m * d_in + c);
      T[m * r + i] = s * acc;
    }
  }
}

/* Backward of the same layer for upstream gradient dY [M, d_out]:
 *   U  = s dY B          [M, r]   (gradient reaching the LoRA bottleneck)
 *   T  = D(X) A^T        [M, r]
 *   dX = dY Wh + D'(U A) (listed rows only; D' = keep / (1 - p), the
 *                         derivative of the dropout map, 1 without dropout)
 *   dA = U^T D(X)        [r, d_in]
 *   dB = s dY^T T        [d_out, r]
 * The frozen base contributes to dX but receives no gradient [QP §2.4].
 * Every sum runs over its index in ascending order; the loops are nested so
 * that the innermost one walks memory contiguously, which changes no sum's
 * order. */
void orc_linear_bwd(const float *Wh, const float *X, const float *dY,
                    const float *A, const float *B, int64_t M, int64_t d_out,
                    int64_t d_in, int64_t r, double s, const int64_t *rows,
                    int64_t nrows, const uint8_t *keep, double keep_prob,
                    double *dX, double *dA, double *dB) {
  double *U = (double *)calloc((size_t)(M * r + 1), sizeof(double));
  double *T = (double *)calloc((size_t)(M * r + 1), sizeof(double));
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    double *u = U + m * r;                     /* u[i] = sum over o of dY[m, o] B[o, i] */
    for (int64_t o = 0; o < d_out; ++o)
      for (int64_t i = 0; i < r; ++i) u[i] += (double)dY[m * d_out + o] * B[o * r + i];
    for (int64_t i = 0; i < r; ++i) {
      double t = 0.0;
      for (int64_t c = 0; c < d_in; ++c)
        t += lora_input(X, keep, keep_prob, m * d_in + c) * A[i * d_in + c];
      u[i] = s * u[i];
      T[m * r + i] = t;
    }
  }
  if (dX) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t k = 0; k < nrows; ++k) {
      int64_t m = rows[k];
      double *base = (double *)calloc((size_t)(d_in > 0 ? d_in : 1), sizeof(double));
      for (int64_t o = 0; o < d_out; ++o)      /* base[c] = sum over o of dY[m, o] Wh[o, c] */
        for (int64_t c = 0; c < d_in; ++c) base[c] += (double)dY[m * d_out + o] * Wh[o * d_in + c];
      for (int64_t c = 0; c < d_in; ++c) {
        double lora = 0.0;
        for (int64_t i = 0; i < r; ++i) lora += U[m * r + i] * A[i * d_in + c];
        if (keep) lora = keep[m * d_in + c] ? lora / keep_prob : 0.0;
        dX[k * d_in + c] = base[c] + lora;
      }
      free(base);
    }
  }
  if (dA) {      /* dA[i, c] = sum over m ascending of U[m, i] D(X)[m, c] */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < r; ++i) {
      double *row = dA + i * d_in;
      for (int64_t c = 0; c < d_in; ++c) row[c] = 0.0;
      for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < d_in; ++c)
          row[c] += U[m * r + i] * lora_input(X, keep, keep_prob, m * d_in + c);
    }
  }
  if (dB) {      /* dB[o, i] = s * sum over m ascending of dY[m, o] T[m, i] */
#pragma omp parallel for schedule(static)
    for (int64_t o0 = 0; o0 < d_out; o0 += 64) {
      const int64_t o1 = o0 + 64 < d_out ? o0 + 64 : d_out;
      for (int64_t o = o0; o < o1; ++o)
        for (int64_t i = 0; i < r; ++i) dB[o * r + i] = 0.0;
      for (int64_t m = 0; m < M; ++m)
        for (int64_t o = o0; o < o1; ++o)
          for (int64_t i = 0; i < r; ++i) dB[o * r + i] += (double)dY[m * d_out + o] * T[m * r + i];
      for (int64_t o = o0; o < o1; ++o)
        for (int64_t i = 0; i < r; ++i) dB[o * r + i] = s * dB[o * r + i];
    }
  }
  free(U);
  free(T);
}

/* ------------------------------------------------------------------------
 * The dropout mask of the LoRA branch [QP §6.3] from a counter-based
 * generator, so that the backward can regenerate the forward's mask from
 * (seed, offset) alone: Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O.
 * Dror, D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11).
 *
 * One round maps counter (c0, c1, c2, c3) under key (k0, k1) to
 *   (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
 * with M0 = 0xD2511F53, M1 = 0xCD9E8D57 and hi/lo the halves of the 64-bit
 * product; the key grows by (0x9E3779B9, 0xBB67AE85) between rounds.
 * ---------------------------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    const uint32_t n3 = (uint32_t)p0;
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

/* keep[m, k] for a row-major [M, d] input: element (m, k) takes word m % 4
 * of Philox4x32-10 at counter (k, floor(m / 4), offset_lo, offset_hi) under
 * key (seed_lo, seed_hi), and is kept when that word u satisfies
 * u >= floor(p * 2^32), so it is dropped with probability p (to 2^-32). */
void orc_dropout_keep(int64_t M, int64_t d, float p, uint64_t seed, uint64_t offset,
                      uint8_t *keep) {
  const uint32_t thr = (uint32_t)floor((double)p * 4294967296.0);
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t k = 0; k < d; ++k) {
      const uint32_t ctr[4] = {(uint32_t)k, (uint32_t)(m / 4), (uint32_t)offset,
                               (uint32_t)(offset >> 32)};
      uint32_t out[4];
      orc_philox4x32_10(ctr, key, out);
      keep[m * d + k] = out[m % 4] >= thr ? 1 : 0;
    }
  }
}

void orc_merge(const float *Wh, const float *A, const float *B, int64_t d_out,
               int64_t d_in, int64_t r, float s, float *Wm) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < d_out; ++n) {
    for (int64_t k = 0; k < d_in; ++k) {
      double dot = 0.0;
      for (int64_t i = 0; i < r; ++i) dot += (double)B[n * r + i] * (double)A[i * d_in + k];
      Wm[n * d_in + k] = (float)((double)Wh[n * d_in + k] + (double)s * dot);
    }
  }
}

/* ------------------------------------------------------------------------
 * Optimizer step on the LoRA factors [QP §7.3] (AdamW, one first and one
 * second moment per parameter, 32-bit) with optional clipping by the global
 * gradient norm [QP §10.2].
 * Readings (the pages strip the formulas):
 *   - AdamW with decoupled weight decay, bias-corrected moments;
 *   - the norm's sum of squares is taken per tensor in groups of 256 by the
 *     stride-halving tree and then by the same tree over the group sums
 *     (the order of the scale mean above), tensors added in list order;
 *   - clip coefficient c = min(1, max_norm / (norm + 1e-6)),
 *     norm = FP32(sqrt(S));
 *   - FP32 element update, each operation rounded on its own in the order
 *     written below; bc_i = FP32(1 - beta_i^step) from an FP64 power.
 * ---------------------------------------------------------------------- */
double orc_sumsq(const float *g, int64_t n) {
  int64_t G = (n + ORC_GROUP - 1) / ORC_GROUP;
  int64_t Gp = 1;
  while (Gp < G) Gp *= 2;
  double *part = (double *)calloc((size_t)Gp, sizeof(double));
  double grp[ORC_GROUP];
  for (int64_t q = 0; q < G; ++q) {
    for (int j = 0; j < ORC_GROUP; ++j) {
      int64_t i = q * ORC_GROUP + j;
      double x = (i < n) ? (double)g[i] : 0.0;
      grp[j] = x * x;
    }
    part[q] = tree_sum(grp, ORC_GROUP);
  }
  double S = tree_sum(part, Gp);
  free(part);
  return S;
}

float orc_clip_coef(double S, float max_norm) {
  float norm = (float)sqrt(S);
  float c = max_norm / (norm + 1e-6f);
  return c < 1.0f ? c : 1.0f;
}

void orc_adamw(float *p, uint16_t *p16, const float *g, float *m, float *v,
               int64_t n, float lr, float beta1, float beta2, float eps,
               float wd, int64_t step, float c) {
  const float lrwd = lr * wd;
  const float ob1 = 1.0f - beta1, ob2 = 1.0f - beta2;
  const float bc1 = (float)(1.0 - pow((double)beta1, (double)step));
  const float bc2 = (float)(1.0 - pow((double)beta2, (double)step));
  for (int64_t i = 0; i < n; ++i) {
    float gi = g[i] * c;
    float pi = p[i];
    pi = pi - lrwd * pi;
    float mi = beta1 * m[i] + ob1 * gi;
    float vi = beta2 * v[i] + ob2 * (gi * gi);
    float mh = mi / bc1;
    float den = sqrtf(vi / bc2) + eps;
    pi = pi - lr * (mh / den);
    p[i] = pi;
    m[i] = mi;
    v[i] = vi;
    if (p16) p16[i] = orc_bf16_rne(pi);
  }
}

void orc_map_nf4_index(const float *x, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_nf4_index(x[i]);
}

void orc_map_fp8_encode(const float *y, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(y[i]);
}

void orc_map_bf16_rne(const float *x, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}

/* Threads the OpenMP loops above use (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int orc_num_threads(void) { return 1; }
void orc_set_num_threads(int n) { (void)n; }
#endif
