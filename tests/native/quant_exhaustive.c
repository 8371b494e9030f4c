/* Exhaustive host check of the division-free INT4 activation quantizer.
 *
 * Definition (SVDQuant technical review, sec. 2.2 Eq.(1), with the readings
 * ties-to-even, codes in [-Q, Q], scale s = fp16(fl32(amax / Q)) saturated,
 * code 0 when s = 0; Q = 7 for INT4, 127 for the 8-bit setting):
 *     code = clamp(round_half_even(fl32(v / s)), -Q, Q)
 * Division-free form evaluated by the activation kernels:
 *     rc = fl32(1 / s); p = fl32(v * rc); e = fma(-p, s, v); q1 = fma(e, rc, p)
 *     q  = med3(q1, -Q, Q);  code bits = bits(fl32(q + 1.5 * 2^23)) & mask
 *     (mask 0xF: the nibble; 0xFF: the byte)
 *
 * Every pair the kernel can meet is enumerated: every positive finite bf16
 * group maximum A (with its scale s(A), supplied by the caller as fp16 bits
 * because this compiler has no _Float16) and every bf16 value v with
 * |v| <= A, both signs.  Prints "pairs mismatches ties nan" and exits 1 on any
 * mismatch or NaN.
 *
 * Usage: quant_exhaustive <table.bin> <Q> [nocorr]
 *   table.bin: 32768 uint16, s(A) = fp16(fl32(A / Q)) bits for every bf16 A;
 *   Q:         7 or 127;
 *   nocorr:    drop the correction step (a planted mistake the check must see).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16_to_float(uint32_t b) {
  uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float half_to_float(uint32_t h) {
  const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);              /* subnormal (exact) */
  else v = ldexpf((float)(m | 0x400), (int)e - 25);   /* normal (exact) */
  return (h & 0x8000) ? -v : v;
}

static uint32_t float_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(int argc, char** argv) {
  if (argc != 3 && argc != 4) return 2;
  const int Q = atoi(argv[2]);
  if (Q != 7 && Q != 127) return 2;
  const float QF = (float)Q;
  const uint32_t mask = Q == 7 ? 0xFu : 0xFFu;
  const int corr = !(argc == 4 && strcmp(argv[3], "nocorr") == 0);
  static uint16_t tab[32768];
  FILE* fp = fopen(argv[1], "rb");
  if (!fp || fread(tab, 2, 32768, fp) != 32768) return 2;
  fclose(fp);
  long long pairs = 0, bad = 0, ties = 0, nans = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad, ties, nans)
  for (int A = 1; A <= 0x7F7F; ++A) {         /* positive finite bf16 maxima */
    const float s = half_to_float(tab[A]);
    const float rc = s > 0.0f ? 1.0f / s : 0.0f;
    for (int vb = 0; vb <= A; ++vb) {           /* 0 <= v <= A (bf16 order = bit order) */
      for (int sg = 0; sg < 2; ++sg) {
        const float v = sg ? -bf16_to_float((uint32_t)vb) : bf16_to_float((uint32_t)vb);
        /* definition */
        int code = 0;
        if (s > 0.0f) {
          const float d = v / s;
          float rq = nearbyintf(d);              /* default mode: ties to even */
          if (fabsf(d - truncf(d)) == 0.5f) ++ties;
          if (rq > QF) rq = QF;
          if (rq < -QF) rq = -QF;
          code = (int)rq;
        }
        /* division-free form */
        const float p = v * rc;
        const float e = fmaf(-p, s, v);
        const float q1 = corr ? fmaf(e, rc, p) : p;
        if (isnan(q1)) ++nans;
        const float q = fminf(fmaxf(q1, -QF), QF);
        const uint32_t bits = float_bits(q + 12582912.0f) & mask;
        if (bits != ((uint32_t)code & mask)) ++bad;
        ++pairs;
      }
    }
  }
  printf("%lld %lld %lld %lld\n", pairs, bad, ties, nans);
  return (bad || nans) ? 1 : 0;
}
