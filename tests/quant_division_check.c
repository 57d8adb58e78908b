// Exhaustive check of the Q quantizer's quotient (test infrastructure). For every finite bf16 /
// fp16 block maximum amax > 0 and every x of the same type with |x| <= amax (both signs, both
// zeros): s = fp32(amax / 448). Where the quantizer takes its short path (2^-96 <= s, finite),
// y_fast = copysign(fma(fma(-q0, s, x), r, q0), x) with r = 1/s and q0 = x * r (all fp32,
// round to nearest even, subnormals kept) must give the same E4M3FN code, after clipping to
// +-448, as the IEEE quotient x / s; fp16 inputs must also give the same fp32 bits. Prints the
// counts; exit status 0 when nothing differs. Build with gcc -O2 -ffp-contract=off (fmaf must be
// one rounding: hardware FMA or libm's).
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bf16(uint16_t h) { return f_of((uint32_t)h << 16); }
static float fp16(uint16_t h) {
  const int e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}
static float e4m3(float y) {
  float a = fabsf(y); if (a > 448.0f) a = 448.0f;
  int e; frexpf(a, &e); int k = (e - 1) - 3; if (k < -9) k = -9;
  float q = a == 0.0f ? 0.0f : ldexpf(rintf(ldexpf(a, -k)), k);
  if (q > 448.0f) q = 448.0f; return copysignf(q, y);
}
int main(void) {
  const float thr = ldexpf(1.0f, -96);
  int fail = 0;
  for (int t = 0; t < 2; t++) {
    const uint16_t maxbits = t == 0 ? 0x7F7F : 0x7BFF;
    long long pairs = 0, bits_bad = 0, code_bad = 0, slow = 0;
    #pragma omp parallel for schedule(dynamic, 64) reduction(+:pairs, bits_bad, code_bad, slow)
    for (int ab = 1; ab <= maxbits; ab++) {
      const float amax = t == 0 ? bf16((uint16_t)ab) : fp16((uint16_t)ab);
      const float s = amax / 448.0f;
      if (!(s >= thr && isfinite(s))) { slow += 2LL * (ab + 1); continue; }
      const float r = 1.0f / s;
      for (int xb = 0; xb <= ab; xb++) {
        for (int sg = 0; sg < 2; sg++) {
          const uint16_t h = (uint16_t)(xb | (sg ? 0x8000 : 0));
          const float x = t == 0 ? bf16(h) : fp16(h);
          const float ex = x / s;
          const float q0 = x * r;
          const float e = fmaf(-q0, s, x);
          const float y = copysignf(fmaf(e, r, q0), x);
          pairs++;
          if (u_of(y) != u_of(ex)) bits_bad++;
          if (u_of(e4m3(y)) != u_of(e4m3(ex))) code_bad++;
        }
      }
    }
    printf("%s: fast-path pairs %lld: fp32 quotients differing %lld, E4M3 codes differing %lld; pairs left to the IEEE division %lld\n",
           t == 0 ? "bf16" : "fp16", pairs, bits_bad, code_bad, slow);
    fail |= code_bad != 0 || (t == 1 && bits_bad != 0);
  }
  return fail;
}
