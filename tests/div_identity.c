/* The encoders' division x / s, as the append kernel computes it:
 *   r = RN(1 / s); y = clamp(RN(x r), -2^80, 2^80); e = fma(-y, s, x);
 *   q = copysign(fma(e, r, y), x)
 * compared with the IEEE quotient RN(x / s).  They must agree bit for bit
 * wherever the quotient can decide a code: |q| >= 2^-20 and below 2^70
 * (every code rounds smaller magnitudes to a signed zero and saturates
 * beyond), with the sign always equal.  Domain: every finite bf16 x against
 * every 31st positive fp16 scale, every UE4M3 scale and 300 per-tensor
 * scales in [2^-30, 2^30]; random fp32 x against the same scales. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float f16_value(int h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
}
static float ue4m3_value(int c) {
  const int e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
}

static long long bad = 0, checks = 0;
static void check(float x, float s, float r) {
  float y = x * r;
  y = fminf(fmaxf(y, -0x1p80f), 0x1p80f);
  const float e = fmaf(-y, s, x);
  const float q = copysignf(fmaf(e, r, y), x);
  const float ref = x / s;
  checks++;
  if (to_bits(q) == to_bits(ref)) return;
  const int same_sign = signbit(q) == signbit(ref);
  const int tiny = fabsf(q) < 0x1p-20f && fabsf(ref) < 0x1p-20f;
  const int huge = fabsf(q) >= 0x1p70f && fabsf(ref) >= 0x1p70f;
  if (!(same_sign && !isnan(q) && (tiny || huge))) {
    if (bad < 5) printf("x=%a s=%a q=%a ref=%a\n", x, s, q, ref);
    bad++;
  }
}

int main(void) {
  static float sc[2000];
  int ns = 0;
  for (int h = 1; h < 0x7C00; h += 31) sc[ns++] = f16_value(h);
  for (int c = 1; c < 127; ++c) sc[ns++] = ue4m3_value(c);
  uint64_t st = 0x2545F4914F6CDD1Dull;
#define NEXT() (st ^= st << 13, st ^= st >> 7, st ^= st << 17, st)
  for (int i = 0; i < 300; ++i) {
    const double u = (double)(NEXT() >> 11) / 9007199254740992.0;
    sc[ns++] = (float)ldexp(1.0 + u, (int)(NEXT() % 61) - 31);
  }
  for (int i = 0; i < ns; ++i) {
    const volatile float r = 1.0f / sc[i];
    for (uint32_t b = 0; b < 65536; ++b) {
      const float x = from_bits(b << 16);
      if (isfinite(x)) check(x, sc[i], r);
    }
    for (int n = 0; n < 2000; ++n) {
      const float x = from_bits((uint32_t)NEXT());
      if (isfinite(x)) check(x, sc[i], r);
    }
  }
  printf("%lld checks, %lld disagreements\n", checks, bad);
  return bad != 0;
}
