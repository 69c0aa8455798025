/*
 * CPU oracle for one decode step of gated linear attention (GLA).
 *
 * TEST INFRASTRUCTURE ONLY (see gemv_ref.c): never part of the product path,
 * shares no code with the HIP library.
 *
 * What it computes (TileLang Case Studies, Case D "Background": the GLA
 * decode kernel's single-step recurrence), for each of BH independent
 * (batch, head) pairs:
 *
 *     S_new = diag(exp(gk)) S + outer(k, v)        S, S_new: DK x DV
 *     o     = scale * q^T S_new                    o: DV
 *
 * q, k, gk (DK each) and v (DV) are fp16/bf16 patterns, decoded exactly; the
 * state S is float32 (row i = the DK index, contiguous along DV).  Everything
 * is evaluated in double: exp from the C library, products and sums in
 * double, i ascending.  S_new is rounded once to float32 (nearest-even, the C
 * conversion), o once to the 16-bit dtype.  o uses the unrounded S_new (the
 * definition).  Readings where the pages are silent: the state is float32,
 * o takes the input dtype, scale is a float32 argument.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

double oracle_decode(int dtype, uint16_t bits);
uint16_t oracle_encode(int dtype, double x);

/* S_out may equal S_in (the state updated in place).  Optional outputs
 * (may be NULL): s64 = S_new before rounding (BH*DK*DV doubles), o64 = o
 * before rounding and oabs = |scale| * sum_i |q_i S_new[i][j]| (BH*DV each). */
int oracle_gla_decode(int dtype, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* gk, const float* S_in, int64_t bh, int64_t dk, int64_t dv,
                      float scale, float* S_out, uint16_t* o, double* s64, double* o64,
                      double* oabs) {
  if (bh < 0 || dk < 0 || dv < 0) return -1;
  for (int64_t h = 0; h < bh; ++h) {
    for (int64_t j = 0; j < dv; ++j) {
      double acc = 0.0, aacc = 0.0;
      const double vj = oracle_decode(dtype, v[h * dv + j]);
      for (int64_t i = 0; i < dk; ++i) {
        const double e = exp(oracle_decode(dtype, gk[h * dk + i]));
        const double ki = oracle_decode(dtype, k[h * dk + i]);
        const double qi = oracle_decode(dtype, q[h * dk + i]);
        const int64_t idx = (h * dk + i) * dv + j;
        const double sn = e * (double)S_in[idx] + ki * vj;
        if (s64) s64[idx] = sn;
        S_out[idx] = (float)sn;           /* after S_in[idx] was read */
        acc += qi * sn;
        aacc += fabs(qi * sn);
      }
      const double oj = (double)scale * acc;
      o[h * dv + j] = oracle_encode(dtype, oj);
      if (o64) o64[h * dv + j] = oj;
      if (oabs) oabs[h * dv + j] = fabs((double)scale) * aacc;
    }
  }
  return 0;
}
