/*
 * Exhaustive check of the division-free code quotient of the GPU row quantize.
 *
 * The quantization record of "Atom (mixed-precision block-outlier low-bit quantization for
 * serving)" (Fields "Bits", "Weight group size", "notes") defines a code as the integer
 * nearest x / s for the group scale s, clamped to [-qmax, qmax].  The GPU kernel does not
 * divide: with r = fl32(1 / s) it forms
 *     t = fl32(x * r),  e = fma(-t, s, x),  u = fma(e, r, t)
 * (a Markstein-style correction of the quotient with fused multiply-adds: e is the exact
 * remainder x - t*s rounded once, and u = t + e*r moves t toward x / s) and rounds
 * clamp(u, -qmax, qmax) to the nearest integer, ties to even.
 *
 * This program takes the reachable (scale, largest absmax for that scale) pairs on stdin
 * (binary: int32 qmax, int32 count, then count pairs of uint16 fp16 bit patterns) and, for
 * every fp16 x with |x| <= that absmax (both signs, zero included), compares
 *     rint(clamp(u))          (the kernel's code)
 * with
 *     clamp(rint(fl32(x / s))) (the definition, IEEE division).
 * A zero scale gives r = 0, so t = 0, e = x, u = 0, and the definition gives code 0.
 * For a normal scale (s >= 2^-14) it also checks that rint(u) alone, without the clamp, is
 * the same code: the kernel clamps only where a subnormal scale occurs.
 * Every operation is IEEE binary32 with round to nearest even: fmaf is glibc's correctly
 * rounded fused multiply-add, and the build turns off contraction.
 * Output: "pairs <n> mismatches <m> unclamped_mismatches <u>" and the first few mismatches.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float half_bits_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const int e = (h >> 10) & 31;
  const uint32_t m = h & 1023;
  float v;
  if (e == 0) {
    v = ldexpf((float)m, -24); /* subnormal (or zero): m * 2^-24, exact in binary32 */
  } else {
    v = ldexpf((float)(m | 1024), e - 25); /* normal: (1024 + m) * 2^(e-25) */
  }
  uint32_t b;
  memcpy(&b, &v, 4);
  b |= sign;
  memcpy(&v, &b, 4);
  return v;
}

static float clampf(float v, float q) { return fminf(fmaxf(v, -q), q); }

int main(void) {
  int32_t qmax_i, count;
  if (fread(&qmax_i, 4, 1, stdin) != 1 || fread(&count, 4, 1, stdin) != 1 || count <= 0) {
    fprintf(stderr, "bad header\n");
    return 2;
  }
  uint16_t* pairs = (uint16_t*)malloc((size_t)count * 4);
  if (!pairs || fread(pairs, 4, (size_t)count, stdin) != (size_t)count) {
    fprintf(stderr, "bad body\n");
    return 2;
  }
  const float qmax = (float)qmax_i;
  /* every finite positive fp16 value, ascending */
  static float xs[0x7C00];
  for (int i = 0; i < 0x7C00; ++i) xs[i] = half_bits_to_float((uint16_t)i);

  long long total = 0, bad = 0, bad_nc = 0;
  int shown = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : total, bad, bad_nc)
  for (int p = 0; p < count; ++p) {
    const float s = half_bits_to_float(pairs[2 * p]);
    const float amax = half_bits_to_float(pairs[2 * p + 1]);
    const float r = s > 0.0f ? 1.0f / s : 0.0f;
    for (int i = 0; i < 0x7C00 && xs[i] <= amax; ++i) {
      for (int sg = 0; sg < 2; ++sg) {
        const float x = sg ? -xs[i] : xs[i];
        const float t = fmaf(x, r, 0.0f);
        const float e = fmaf(-t, s, x);
        const float u = fmaf(e, r, t);
        const float code = nearbyintf(clampf(u, qmax));
        const float want = s > 0.0f ? clampf(nearbyintf(x / s), qmax) : 0.0f;
        ++total;
        if (s >= 0x1p-14f && nearbyintf(u) != code) {
          ++bad_nc;
#pragma omp critical
          {
            if (shown < 8) {
              fprintf(stdout, "unclamped mismatch s=%a x=%a u=%a code=%g\n", s, x, u, code);
              ++shown;
            }
          }
        }
        if (code != want) {
          ++bad;
#pragma omp critical
          {
            if (shown < 8) {
              fprintf(stdout, "mismatch s=%a x=%a code=%g want=%g\n", s, x, code, want);
              ++shown;
            }
          }
        }
      }
    }
  }
  printf("pairs %lld mismatches %lld unclamped_mismatches %lld\n", total, bad, bad_nc);
  free(pairs);
  return (bad || bad_nc) ? 1 : 0;
}
