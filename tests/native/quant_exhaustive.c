/* Exhaustive host check of the division-free INT4 activation quantizer.
 *
 * Definition (SVDQuant technical review, sec. 2.2 Eq.(1), with the readings
 * ties-to-even, codes in [-7, 7], scale s = fp16(fl32(amax / 7)) saturated,
 * code 0 when s = 0):
 *     code = clamp(round_half_even(fl32(v / s)), -7, 7)
 * Division-free form evaluated by the activation kernel:
 *     rc = fl32(1 / s); p = fl32(v * rc); e = fma(-p, s, v); q1 = fma(e, rc, p)
 *     q  = med3(q1, -7, 7);  nibble = bits(fl32(q + 1.5 * 2^23)) & 0xF
 *
 * Every pair the kernel can meet is enumerated: every positive finite bf16
 * group maximum A (with its scale s(A), supplied by the caller as fp16 bits
 * because this compiler has no _Float16) and every bf16 value v with
 * |v| <= A, both signs.  Prints "pairs mismatches ties nan" and exits 1 on any
 * mismatch or NaN.
 *
 * Usage: quant_exhaustive <table.bin> [nocorr]
 *   table.bin: 32768 uint16, s(A) as fp16 bits for every bf16 bit pattern A;
 *   nocorr:    drop the correction step (a planted mistake the check must see).
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
  if (argc != 2 && argc != 3) return 2;
  const int corr = !(argc == 3 && strcmp(argv[2], "nocorr") == 0);
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
          if (rq > 7.0f) rq = 7.0f;
          if (rq < -7.0f) rq = -7.0f;
          code = (int)rq;
        }
        /* division-free form */
        const float p = v * rc;
        const float e = fmaf(-p, s, v);
        const float q1 = corr ? fmaf(e, rc, p) : p;
        if (isnan(q1)) ++nans;
        const float q = fminf(fmaxf(q1, -7.0f), 7.0f);
        const uint32_t nib = float_bits(q + 12582912.0f) & 0xFu;
        if (nib != ((uint32_t)code & 0xFu)) ++bad;
        ++pairs;
      }
    }
  }
  printf("%lld %lld %lld %lld\n", pairs, bad, ties, nans);
  return (bad || nans) ? 1 : 0;
}
