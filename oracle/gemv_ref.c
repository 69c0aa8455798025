/*
 * CPU oracle for the dense GEMV  c = B @ a.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * What it computes (TileLang Case Studies, Case B "Background": c = B @ a with
 * B of shape (n, k) row-major and a of shape (k,)):
 *
 *     c[i] = round_to_dtype( sum_{j=0}^{k-1} B[i][j] * a[j] )
 *
 * written out plainly:
 *   1. every 16-bit input is decoded exactly to a double, from the IEEE-754
 *      binary16 definition (fp16) or the bfloat16 definition (the top half of
 *      an IEEE-754 binary32);
 *   2. the products are formed in double (exact: at most 22 significant
 *      bits) and summed in double, j ascending, next to the sum of their
 *      absolute values;
 *   3. the double sum is rounded once, to nearest with ties to even, into the
 *      output dtype (the dtype of the inputs).
 *
 * The pages never state the accumulation precision or the rounding of the
 * output; the accumulation here is fp64 (the plain definition, up to fp64
 * rounding of the sum) and the output rounding is IEEE round-to-nearest-even.
 * Special values follow IEEE-754: NaN in -> NaN out, inf*0 -> NaN,
 * overflow -> inf.  NaN outputs use the canonical quiet NaN (0x7E00 fp16,
 * 0x7FC0 bf16).  Subnormals are honoured on input and output.
 *
 * Plain, single-threaded, slow on purpose.  Build: gcc -O2 -fno-fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define ORACLE_F16 0
#define ORACLE_BF16 1

/* ---- step 1: exact decode ------------------------------------------------ */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   e == 0       : (-1)^s * m * 2^-24            (zero and subnormals)
 *   0 < e < 31   : (-1)^s * (1024 + m) * 2^(e-25)
 *   e == 31      : inf (m == 0) or NaN            */
double oracle_decode_f16(uint16_t h) {
  int s = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 31) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -24);
  } else {
    v = ldexp((double)(1024 + m), e - 25);
  }
  return s ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 *   e == 0       : (-1)^s * m * 2^-133
 *   0 < e < 255  : (-1)^s * (128 + m) * 2^(e-134)
 *   e == 255     : inf (m == 0) or NaN            */
double oracle_decode_bf16(uint16_t b) {
  int s = (b >> 15) & 1;
  int e = (b >> 7) & 255;
  int m = b & 127;
  double v;
  if (e == 255) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -133);
  } else {
    v = ldexp((double)(128 + m), e - 134);
  }
  return s ? -v : v;
}

double oracle_decode(int dtype, uint16_t bits) {
  return dtype == ORACLE_F16 ? oracle_decode_f16(bits) : oracle_decode_bf16(bits);
}

/* ---- step 3: one rounding, nearest-even ---------------------------------- */

/* Generic encoder for a binary format with `fbits` fraction bits, exponent
 * bias `bias` and all-ones exponent `emax_field` reserved for inf/NaN.
 * The value is scaled by the quantum q of its binade (an exact power of two),
 * rounded to an integer with ties to even (rint under the default rounding
 * mode), and re-assembled from the rounded magnitude. */
static uint16_t encode_generic(double x, int fbits, int bias, int emax_field,
                               uint16_t qnan) {
  uint16_t sign = signbit(x) ? (uint16_t)0x8000 : (uint16_t)0;
  if (isnan(x)) return qnan;
  double ax = fabs(x);
  int emin = 1 - bias;                     /* exponent of the smallest normal */
  /* largest finite = (2 - 2^-fbits) * 2^(emax_field-1-bias); values at or
   * above the midpoint to 2^(emax_field-bias) round to inf. */
  double overflow_at = ldexp(2.0 - ldexp(1.0, -(fbits + 1)), emax_field - 1 - bias);
  if (isinf(ax) || ax >= overflow_at) return (uint16_t)(sign | (emax_field << fbits));
  if (ax == 0.0) return sign;
  int ex;
  frexp(ax, &ex);                          /* ax = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;                          /* floor(log2(ax)) */
  if (e < emin) e = emin;                  /* subnormal range: fixed quantum */
  double q = ldexp(1.0, e - fbits);        /* spacing of representable values */
  double m = rint(ax / q);                 /* ties to even */
  double r = m * q;                        /* rounded magnitude */
  if (r >= ldexp(1.0, emax_field - bias)) return (uint16_t)(sign | (emax_field << fbits));
  if (r < ldexp(1.0, emin)) {              /* subnormal (or zero) result */
    return (uint16_t)(sign | (uint16_t)ldexp(r, bias - 1 + fbits));
  }
  frexp(r, &ex);
  int er = ex - 1;
  uint32_t frac = (uint32_t)(ldexp(r, fbits - er) - ldexp(1.0, fbits));
  return (uint16_t)(sign | ((uint32_t)(er + bias) << fbits) | frac);
}

uint16_t oracle_encode_f16(double x) { return encode_generic(x, 10, 15, 31, 0x7E00); }
uint16_t oracle_encode_bf16(double x) { return encode_generic(x, 7, 127, 255, 0x7FC0); }

uint16_t oracle_encode(int dtype, double x) {
  return dtype == ORACLE_F16 ? oracle_encode_f16(x) : oracle_encode_bf16(x);
}

/* ---- array helpers (for the pins) ---------------------------------------- */

void oracle_decode_array(int dtype, const uint16_t* bits, double* out, int64_t count) {
  for (int64_t i = 0; i < count; ++i) out[i] = oracle_decode(dtype, bits[i]);
}

void oracle_encode_array(int dtype, const double* x, uint16_t* out, int64_t count) {
  for (int64_t i = 0; i < count; ++i) out[i] = oracle_encode(dtype, x[i]);
}

/* ---- the GEMV ------------------------------------------------------------ */

/* With an epilogue (page "Optimizing TileLang Programs", epilogue fusion:
 * post-operations applied before the single write of the result):
 *     c[i] = round_to_dtype( alpha * sum_j B[i][j] a[j] + bias[i] )
 * alpha is a float32 value (exact in double), bias[i] a `dtype` value (exact
 * in double); the expression is evaluated in double and rounded once. */
int oracle_gemv_epilogue(int dtype, const uint16_t* B, const uint16_t* a, int64_t n, int64_t k,
                         float alpha, const uint16_t* bias, uint16_t* c, double* s,
                         double* abs_out, double* a_scratch);

/* B: n*k 16-bit patterns, row-major (row i starts at B + i*k).
 * a: k patterns.  Outputs, per row i:
 *   c[i]   rounded result (16-bit pattern of `dtype`),
 *   s[i]   the fp64 sum before rounding (may be NULL),
 *   abs[i] sum_j |B[i][j] * a[j]| in fp64 (may be NULL).
 * k == 0 gives the empty sum, +0.  Returns 0, or -1 on a bad argument. */
int oracle_gemv(int dtype, const uint16_t* B, const uint16_t* a, int64_t n, int64_t k,
                uint16_t* c, double* s, double* abs_out, double* a_scratch) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  if (n < 0 || k < 0) return -1;
  /* decode a once (a_scratch holds k doubles) */
  for (int64_t j = 0; j < k; ++j) a_scratch[j] = oracle_decode(dtype, a[j]);
  for (int64_t i = 0; i < n; ++i) {
    const uint16_t* row = B + i * k;
    double sum = 0.0, asum = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      double p = oracle_decode(dtype, row[j]) * a_scratch[j];
      sum += p;
      asum += fabs(p);
    }
    c[i] = oracle_encode(dtype, sum);
    if (s) s[i] = sum;
    if (abs_out) abs_out[i] = asum;
  }
  return 0;
}

int oracle_gemv_epilogue(int dtype, const uint16_t* B, const uint16_t* a, int64_t n, int64_t k,
                         float alpha, const uint16_t* bias, uint16_t* c, double* s,
                         double* abs_out, double* a_scratch) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  if (n < 0 || k < 0) return -1;
  for (int64_t j = 0; j < k; ++j) a_scratch[j] = oracle_decode(dtype, a[j]);
  for (int64_t i = 0; i < n; ++i) {
    const uint16_t* row = B + i * k;
    double sum = 0.0, asum = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      double p = oracle_decode(dtype, row[j]) * a_scratch[j];
      sum += p;
      asum += fabs(p);
    }
    double y = (double)alpha * sum;
    if (bias) y += oracle_decode(dtype, bias[i]);
    c[i] = oracle_encode(dtype, y);
    if (s) s[i] = y;
    if (abs_out) abs_out[i] = asum;
  }
  return 0;
}
