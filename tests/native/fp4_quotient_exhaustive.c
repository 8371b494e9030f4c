/* Exhaustive host check of the division-free quotient of the FP4 (NVFP4)
 * activation quantizer.
 *
 * Definition (reading R20 of the SVDQuant technical review's NVFP4 setting,
 * sec. 8): with block scale S = sb * 2^k (sb an FP8 E4M3 value, 2^k the
 * power-of-two tensor scale), code = E2M1_RNE_sat(fl32(v / S)), ties to the
 * even code, sign of the quotient in bit 3.
 * Division-free form evaluated by the activation kernel:
 *     rc = fl32(1 / S); p = fl32(v * rc); e = fma(-p, S, v); q1 = fma(e, rc, p)
 *     y  = copysign(|v| <= 8 S ? q1 : 8, v)
 * (the copysign keeps the quotient's sign where q1 loses it: v = -0 gives
 * e = 0 and q1 = 0 * rc + (-0) = +0).
 * and the code of y (the kernel's hardware conversion rounds to nearest even
 * on the E2M1 grid and saturates; shown by the GPU parity tests).
 *
 * Enumerated: every positive finite E4M3 value sb (bits 0x01..0x7E), every
 * tensor-scale exponent k in [-30, 10], and every finite bf16 value v (both
 * signs, zeros and subnormals included).  Prints "pairs code_mismatches
 * quotient_mismatches" and exits 1 on any code mismatch.  (Quotient bits differ
 * only where |v / S| is far below the first rounding threshold 0.25.)
 *
 * Usage: fp4_quotient_exhaustive [nocorr]   (nocorr: drop the correction step,
 * a planted mistake the check must see)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16_to_float(uint32_t b) {
  uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t float_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* E4M3 value of bits 0x00..0x7E (exact) */
static float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xF, m = b & 7;
  return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), (int)e - 10);
}

/* E2M1 code, threshold form: count of midpoints below |y|, ties to the even code */
static uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  uint32_t idx = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return idx | (signbit(y) ? 8u : 0u);
}

int main(int argc, char** argv) {
  const int corr = !(argc == 2 && strcmp(argv[1], "nocorr") == 0);
  long long pairs = 0, bad = 0, qbad = 0;
  for (int k = -30; k <= 10; ++k) {
#pragma omp parallel for reduction(+ : pairs, bad, qbad) schedule(dynamic)
    for (uint32_t sbb = 1; sbb <= 0x7E; ++sbb) {
      const float S = ldexpf(e4m3_value(sbb), k);   /* exact */
      const float rc = 1.0f / S;
      const float S8 = 8.0f * S;
      for (uint32_t vb = 0; vb < 0x10000; ++vb) {
        const float v = bf16_to_float(vb);
        if (!isfinite(v)) continue;
        const float qd = v / S;                       /* the definition's quotient */
        const float p = v * rc;
        const float e = fmaf(-p, S, v);
        const float q1 = corr ? fmaf(e, rc, p) : p;
        const float y = copysignf(fabsf(v) <= S8 ? q1 : 8.0f, v);
        ++pairs;
        if (e2m1_code(y) != e2m1_code(qd)) ++bad;
        if (fabsf(v) <= S8 && float_bits(copysignf(q1, v)) != float_bits(qd)) {
          ++qbad;
          if (fabsf(qd) >= 0.125f) ++bad;   /* a wrong quotient near a threshold counts as a mismatch */
        }
      }
    }
  }
  printf("%lld %lld %lld\n", pairs, bad, qbad);
  return bad != 0;
}
