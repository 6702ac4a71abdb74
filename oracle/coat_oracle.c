/*
 * coat_oracle.c -- plain, single-threaded CPU reference of COAT's FP8 AdamW
 * step with Dynamic Range Expansion.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the benchmark's
 * CPU-baseline leg; never by the product path.  Written for a reader checking
 * it against the sources by eye: one group at a time, one element at a time,
 * double precision wherever the sources do not fix a precision, FP32 where the
 * optimizer state itself is FP32.  Build with -ffp-contract=off so that the
 * FP32 AdamW arithmetic keeps the equation's literal rounding order.
 *
 * Citations: see coat_oracle.h for [P1] (xllm-io review of COAT, section 三
 * 核心公式) and [OCP] (OFP8 specification, E4M3).
 */
#include "coat_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

/* [OCP] E4M3: largest finite magnitude and smallest normal magnitude. */
static const double kE4M3Max = 448.0;
static const double kE4M3MinNormal = 0.015625; /* 2^-6 */
/* Reading: upper clamp of the expansion exponent. */
static const double kMaxK = 16.0;

/* [P1] eq. for the optimal k needs R_E4M3; taken as max / min-normal. */
static double e4m3_log2_range(void) { return log2(kE4M3Max / kE4M3MinNormal); }

/* ---------------------------------------------------------------- codec */

/* [OCP] E4M3 layout: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa.  Exponent field 0 encodes subnormals mant * 2^-9; S.1111.111 is
 * NaN; there is no infinity. */
double coat_oracle_e4m3_decode(uint8_t code) {
  const int sign = (code >> 7) & 1;
  const int e = (code >> 3) & 0xF;
  const int f = code & 7;
  double mag;
  if (e == 15 && f == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)f, -9);
  else
    mag = ldexp(1.0 + f / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Round a nonnegative real y to an integer, ties to the even integer. */
static double round_half_even(double y) {
  const double lo = floor(y);
  const double frac = y - lo;
  if (frac > 0.5) return lo + 1.0;
  if (frac < 0.5) return lo;
  return (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
}

/* [OCP] nearest representable E4M3 magnitude, ties to even, saturating at the
 * largest finite value (the method never asks for more than 448). */
uint8_t coat_oracle_e4m3_encode(double x) {
  if (isnan(x)) return 0x7F;
  const uint8_t sign = (x < 0) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a > kE4M3Max) a = kE4M3Max;
  /* Spacing of representable values around a: 2^-9 below the smallest
   * normal, else 2^(exponent - 3) for the 3 mantissa bits. */
  double quantum;
  if (a < kE4M3MinNormal) {
    quantum = ldexp(1.0, -9);
  } else {
    int ex;
    frexp(a, &ex); /* a = fr * 2^ex, fr in [0.5, 1) */
    quantum = ldexp(1.0, (ex - 1) - 3);
  }
  const double units = round_half_even(a / quantum); /* exact division */
  const double v = units * quantum;                   /* nearest value  */
  /* Encode the representable value v (v <= 448, so no overflow). */
  uint8_t mag;
  if (v < kE4M3MinNormal) {
    mag = (uint8_t)(v / ldexp(1.0, -9)); /* subnormal (or zero) code */
  } else {
    int ex;
    const double fr = frexp(v, &ex);
    const int e_unbiased = ex - 1;
    const int f = (int)((2.0 * fr - 1.0) * 8.0); /* exact: v is on the grid */
    mag = (uint8_t)(((e_unbiased + 7) << 3) | f);
  }
  return (uint8_t)(sign | mag);
}

void coat_oracle_e4m3_encode_array(const double* x, int64_t n, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = coat_oracle_e4m3_encode(x[i]);
}

void coat_oracle_e4m3_decode_array(const uint8_t* codes, int64_t n, double* x) {
  for (int64_t i = 0; i < n; ++i) x[i] = coat_oracle_e4m3_decode(codes[i]);
}

/* ------------------------------------------------------- group quantizer */

/* Statistics of one group ([P1] eq. for R_X): max |x| and the smallest
 * nonzero |x| (reading: zeros are left out; none means the group is empty). */
static void group_stats(const float* x, int64_t len, float* smax, float* smin_nz) {
  float s = 0.0f;
  float mu = INFINITY;
  for (int64_t i = 0; i < len; ++i) {
    const float a = fabsf(x[i]);
    if (a > s) s = a;
    if (a != 0.0f && a < mu) mu = a;
  }
  *smax = s;
  *smin_nz = mu;
}

/* [P1] eq. for the optimal k: (R_X)^k = R_E4M3, so k = log2(R_E4M3)/log2(R_X).
 * Reading: R_X = 1 (nothing to expand) and any larger k are clamped to 16. */
static double expansion_exponent(float smax, float smin_nz) {
  const double lx = log2((double)smax / (double)smin_nz);
  if (lx == 0.0) return kMaxK;
  const double k = e4m3_log2_range() / lx;
  return (k < kMaxK) ? k : kMaxK;
}

/* Quantize one group: f(x) = sign(x)|x|^k ([P1] eq. f), then the absmax
 * quantizer Q ([P1] eq. FP8量化) of f(X) with round-to-nearest-even.
 * Since max|f(X)| = s^k, the code of x is RNE(448 * (|x|/s)^k); the group
 * stores s itself as its scale (reading) and k as FP32. */
static void quantize_group(const float* x, int64_t len, int dre, uint8_t* codes,
                           float* scale, float* kout, double* q_out) {
  float s, mu;
  group_stats(x, len, &s, &mu);
  if (s == 0.0f) { /* empty group (reading): scale 0, k 1, codes 0 */
    *scale = 0.0f;
    *kout = 1.0f;
    for (int64_t i = 0; i < len; ++i) {
      codes[i] = 0x00;
      if (q_out) q_out[i] = 0.0;
    }
    return;
  }
  const float kf = dre ? (float)expansion_exponent(s, mu) : 1.0f;
  *scale = s;
  *kout = kf;
  for (int64_t i = 0; i < len; ++i) {
    double q = kE4M3Max * pow(fabs((double)x[i]) / (double)s, (double)kf);
    if (q > kE4M3Max) q = kE4M3Max;
    if (q_out) q_out[i] = q;
    uint8_t c = coat_oracle_e4m3_encode(q);
    if (x[i] < 0.0f) c |= 0x80; /* sign of f(x) is the sign of x */
    codes[i] = c;
  }
}

/* Dequantize one group: invert Q (multiply back by the scale, here folded into
 * s) and then invert f: x = sign(c) * s * (|c|/448)^(1/k). */
static int dequantize_group(const uint8_t* codes, int64_t len, float scale,
                            float k, float* x) {
  if (scale == 0.0f) { /* empty group: every value is zero, k ignored */
    for (int64_t i = 0; i < len; ++i) x[i] = 0.0f;
    return COAT_ORACLE_OK;
  }
  if (!(k > 0.0f) || !(scale > 0.0f)) return COAT_ORACLE_ESTATE;
  for (int64_t i = 0; i < len; ++i) {
    const uint8_t c = codes[i];
    if ((c & 0x7F) == 0x7F) return COAT_ORACLE_ESTATE; /* NaN code */
    const double mag = coat_oracle_e4m3_decode((uint8_t)(c & 0x7F));
    if (mag == 0.0) {
      x[i] = 0.0f;
      continue;
    }
    const double val = (double)scale * pow(mag / kE4M3Max, 1.0 / (double)k);
    x[i] = (float)((c & 0x80) ? -val : val);
  }
  return COAT_ORACLE_OK;
}

int coat_oracle_expand_quantize(const float* x, int64_t n, int32_t group_size,
                                int32_t dre, uint8_t* codes, float* scale,
                                float* k, double* q_out) {
  if (n < 0 || group_size < 1) return COAT_ORACLE_EINVAL;
  for (int64_t g0 = 0, gi = 0; g0 < n; g0 += group_size, ++gi) {
    const int64_t len = (n - g0 < group_size) ? (n - g0) : group_size;
    quantize_group(x + g0, len, dre, codes + g0, scale + gi, k + gi,
                   q_out ? q_out + g0 : NULL);
  }
  return COAT_ORACLE_OK;
}

int coat_oracle_dequantize_expand(const uint8_t* codes, const float* scale,
                                  const float* k, int64_t n, int32_t group_size,
                                  float* x) {
  if (n < 0 || group_size < 1) return COAT_ORACLE_EINVAL;
  for (int64_t g0 = 0, gi = 0; g0 < n; g0 += group_size, ++gi) {
    const int64_t len = (n - g0 < group_size) ? (n - g0) : group_size;
    const int rc = dequantize_group(codes + g0, len, scale[gi], k[gi], x + g0);
    if (rc != COAT_ORACLE_OK) return rc;
  }
  return COAT_ORACLE_OK;
}

/* ------------------------------------------------------------------ AdamW */

/* BF16 is the upper half of an FP32 bit pattern, so widening is exact. */
static float bf16_to_float(uint16_t b) {
  union { uint32_t u; float f; } cv;
  cv.u = (uint32_t)b << 16;
  return cv.f;
}

typedef struct {
  float lr, beta1, beta2, eps, wd;
  float one_minus_b1, one_minus_b2; /* (1 - beta) in FP32 */
  float bc1, bc2;                   /* 1 - beta^t, from double, as FP32 */
} adamw_consts;

static int make_consts(float lr, float beta1, float beta2, float eps, float wd,
                       int64_t step, adamw_consts* c) {
  if (step < 1 || !(beta1 >= 0.0f && beta1 < 1.0f) ||
      !(beta2 >= 0.0f && beta2 < 1.0f) || !isfinite(lr) || !isfinite(eps) ||
      !isfinite(wd))
    return COAT_ORACLE_EINVAL;
  c->lr = lr;
  c->beta1 = beta1;
  c->beta2 = beta2;
  c->eps = eps;
  c->wd = wd;
  c->one_minus_b1 = 1.0f - beta1;
  c->one_minus_b2 = 1.0f - beta2;
  c->bc1 = (float)(1.0 - pow((double)beta1, (double)step));
  c->bc2 = (float)(1.0 - pow((double)beta2, (double)step));
  return COAT_ORACLE_OK;
}

/* [P1] eq. AdamW for one element, FP32, in the equation's order:
 *   m_t = b1 m + (1-b1) g ;  v_t = b2 v + (1-b2) g^2
 *   mh = m_t / (1-b1^t)   ;  vh = v_t / (1-b2^t)
 *   w  = w - lr (mh / (sqrt(vh) + eps) + wd w)                              */
static void adamw_element(const adamw_consts* c, float g, float* w, float* m,
                          float* v) {
  const float mt = c->beta1 * (*m) + c->one_minus_b1 * g;
  const float vt = c->beta2 * (*v) + c->one_minus_b2 * (g * g);
  const float mh = mt / c->bc1;
  const float vh = vt / c->bc2;
  const float denom = sqrtf(vh) + c->eps;
  *w = *w - c->lr * (mh / denom + c->wd * (*w));
  *m = mt;
  *v = vt;
}

int coat_oracle_adamw_step_fp32(float* w, const uint16_t* grad_bf16, float* m,
                                float* v, int64_t n, float lr, float beta1,
                                float beta2, float eps, float weight_decay,
                                int64_t step) {
  adamw_consts c;
  if (n < 0) return COAT_ORACLE_EINVAL;
  const int rc = make_consts(lr, beta1, beta2, eps, weight_decay, step, &c);
  if (rc != COAT_ORACLE_OK) return rc;
  for (int64_t i = 0; i < n; ++i)
    adamw_element(&c, bf16_to_float(grad_bf16[i]), &w[i], &m[i], &v[i]);
  return COAT_ORACLE_OK;
}

/* Fused step, one group at a time ([P1] section 四: the optimizer state
 * update is a single fused pass; reading for the order): dequantize m and v
 * (inverse of Q, then of f), AdamW on the FP32 values, then expand and
 * quantize the new moments with freshly computed per-group k and scale. */
int coat_oracle_adamw_fp8_step(float* w, const uint16_t* grad_bf16,
                               uint8_t* m_codes, float* m_scale, float* m_k,
                               uint8_t* v_codes, float* v_scale, float* v_k,
                               int64_t n, int32_t group_size, int32_t dre,
                               float lr, float beta1, float beta2, float eps,
                               float weight_decay, int64_t step, float* m_out,
                               float* v_out, double* qm_out, double* qv_out) {
  adamw_consts c;
  if (n < 0 || group_size < 1) return COAT_ORACLE_EINVAL;
  int rc = make_consts(lr, beta1, beta2, eps, weight_decay, step, &c);
  if (rc != COAT_ORACLE_OK) return rc;
  float* mg = (float*)malloc(sizeof(float) * (size_t)group_size);
  float* vg = (float*)malloc(sizeof(float) * (size_t)group_size);
  if (!mg || !vg) {
    free(mg);
    free(vg);
    return COAT_ORACLE_EINVAL;
  }
  for (int64_t g0 = 0, gi = 0; g0 < n; g0 += group_size, ++gi) {
    const int64_t len = (n - g0 < group_size) ? (n - g0) : group_size;
    rc = dequantize_group(m_codes + g0, len, m_scale[gi], m_k[gi], mg);
    if (rc == COAT_ORACLE_OK)
      rc = dequantize_group(v_codes + g0, len, v_scale[gi], v_k[gi], vg);
    if (rc != COAT_ORACLE_OK) break;
    for (int64_t i = 0; i < len; ++i)
      adamw_element(&c, bf16_to_float(grad_bf16[g0 + i]), &w[g0 + i], &mg[i],
                    &vg[i]);
    if (m_out)
      for (int64_t i = 0; i < len; ++i) m_out[g0 + i] = mg[i];
    if (v_out)
      for (int64_t i = 0; i < len; ++i) v_out[g0 + i] = vg[i];
    quantize_group(mg, len, dre, m_codes + g0, m_scale + gi, m_k + gi,
                   qm_out ? qm_out + g0 : NULL);
    quantize_group(vg, len, dre, v_codes + g0, v_scale + gi, v_k + gi,
                   qv_out ? qv_out + g0 : NULL);
  }
  free(mg);
  free(vg);
  return rc;
}

/* --------------------------------------------- activation quantizer (1xG) */

/* One 1xG group through [P1] eq. FP8量化: S = max|X| / 448 and
 * X_FP8 = round(X / S), rounding to nearest with ties to even (reading).
 * The code is decided on the exact quotient X / S = 448 x / max.  In double,
 * 448 x is exact (an FP32 x has 24 significant bits) and the one division by
 * max rounds to 53 bits.  That rounding cannot move the quotient across an
 * E4M3 midpoint, nor onto one: a midpoint has 5 significant bits, so
 * 448 x - midpoint * max is either zero or at least 2^-30 of either term,
 * far above 2^-53.  Hence the double quotient rounds to the same E4M3 value
 * as the exact one.  The sign is that of x (a negative value that rounds to
 * zero keeps it: 0x80); -0.0 and zero give 0x00.  The stored scale is S
 * rounded once to FP32.  An all-zero group stores S = 0 and codes 0. */
static void quantize_group_e4m3(const float* x, int64_t len, uint8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int64_t j = 0; j < len; ++j) {
    const float a = fabsf(x[j]);
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {
    *scale = 0.0f;
    for (int64_t j = 0; j < len; ++j) codes[j] = 0x00;
    return;
  }
  *scale = amax / (float)kE4M3Max;
  for (int64_t j = 0; j < len; ++j) {
    const double q = (kE4M3Max * (double)x[j]) / (double)amax;
    codes[j] = coat_oracle_e4m3_encode(q);
  }
}

int coat_oracle_quantize_act(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                             int32_t group_size, uint8_t* codes, float* scales,
                             uint8_t* codes_t) {
  if (rows < 0 || cols < 0 || group_size < 1 || cols % group_size != 0)
    return COAT_ORACLE_EINVAL;
  const int64_t groups_per_row = cols / group_size;
  float* row = malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
  if (!row) return COAT_ORACLE_ENOMEM;
  for (int64_t i = 0; i < rows; ++i) {
    for (int64_t j = 0; j < cols; ++j) row[j] = bf16_to_float(x_bf16[i * cols + j]);
    for (int64_t gj = 0; gj < groups_per_row; ++gj)
      quantize_group_e4m3(row + gj * group_size, group_size, codes + i * cols + gj * group_size,
                          scales + i * groups_per_row + gj);
  }
  free(row);
  if (codes_t)
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t j = 0; j < cols; ++j) codes_t[j * rows + i] = codes[i * cols + j];
  return COAT_ORACLE_OK;
}

/* ------------------------------------------- group-scaled FP8 linear layer */

/* E4M3 value of a code in units of 2^-9, the smallest subnormal: every finite
 * E4M3 value is an integer multiple of it, so products of two such integers
 * and their sums are exact in int64. */
static int32_t e4m3_units(uint8_t code) {
  return (int32_t)(coat_oracle_e4m3_decode(code) * 512.0);
}

int coat_oracle_gemm_fp8_group_quant(const uint8_t* a, const uint8_t* b, float a_scale,
                                     float b_scale, int64_t M, int64_t N, int64_t K,
                                     int32_t group_size, uint8_t* codes, float* scales,
                                     double* c_exact, float* c_f32) {
  if (M < 0 || N < 0 || K < 0 || K > (1 << 17) || group_size < 1 || N % group_size != 0)
    return COAT_ORACLE_EINVAL;
  for (int64_t i = 0; i < M * K; ++i)
    if ((a[i] & 0x7F) == 0x7F) return COAT_ORACLE_ESTATE;
  for (int64_t i = 0; i < N * K; ++i)
    if ((b[i] & 0x7F) == 0x7F) return COAT_ORACLE_ESTATE;
  int32_t* ia = malloc(sizeof(int32_t) * (size_t)(M * K > 0 ? M * K : 1));
  int32_t* ib = malloc(sizeof(int32_t) * (size_t)(N * K > 0 ? N * K : 1));
  float* row = malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
  if (!ia || !ib || !row) {
    free(ia);
    free(ib);
    free(row);
    return COAT_ORACLE_ENOMEM;
  }
  for (int64_t i = 0; i < M * K; ++i) ia[i] = e4m3_units(a[i]);
  for (int64_t i = 0; i < N * K; ++i) ib[i] = e4m3_units(b[i]);
  const double scale = (double)a_scale * (double)b_scale;  /* exact: 24 + 24 bits */
  const int64_t groups_per_row = N / group_size;
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      /* C = A B^T: the sum over k is exact (|sum| < K * 2^36 <= 2^53). */
      int64_t acc = 0;
      for (int64_t k = 0; k < K; ++k) acc += (int64_t)ia[i * K + k] * ib[j * K + k];
      const double c = (double)acc * 0x1p-18 * scale;
      if (c_exact) c_exact[i * N + j] = c;
      row[j] = (float)c;
    }
    if (c_f32)
      for (int64_t j = 0; j < N; ++j) c_f32[i * N + j] = row[j];
    for (int64_t gj = 0; gj < groups_per_row; ++gj)
      quantize_group_e4m3(row + gj * group_size, group_size, codes + i * N + gj * group_size,
                          scales + i * groups_per_row + gj);
  }
  free(ia);
  free(ib);
  free(row);
  return COAT_ORACLE_OK;
}
