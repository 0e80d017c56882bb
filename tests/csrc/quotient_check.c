/* Host check of the quantizers' quotient: for a scale s >= 1e-30 and r = RN(1/s),
 *   q0 = RN(x r), e = RN(x - q0 s) (fused), q = copysign(RN(q0 + e r) (fused), x)
 * must give the same int8 code (rint, clamp +-127) and the same e4m3fn code as
 * RN(x / s).  Mode "exhaustive": every finite 16-bit value x (fp16 or bf16) and
 * every scale RN(amax / qmax) with amax a 16-bit value >= |x| ("exhaustive N": every
 * N-th such amax).  Mode "random":
 * arbitrary fp32 scales, x uniform in +-qmax s and on exact half-step
 * boundaries and their neighbours.  Exit status 0 when no code differs. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint32_t e4m3(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7f;
  uint32_t sign = (u >> 24) & 0x80u, au = u & 0x7fffffffu;
  float a;
  memcpy(&a, &au, 4);
  a = a > 448.0f ? 448.0f : a;
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    uint32_t b;
    memcpy(&b, &a, 4);
    b += 0x7ffffu + ((b >> 20) & 1u);
    code = (b >> 20) - (120u << 3);
  }
  return code | sign;
}
static int i8(float v) {
  float r = rintf(v);
  r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
  return (int)r;
}
static float quot(float x, float s, float r) {
  if (!(s >= 1e-30f)) return x / s;
  const float q0 = x * r;
  const float e = fmaf(-q0, s, x);
  return copysignf(fmaf(e, r, q0), x);
}
static int differ_r(float x, float s, float r, float qmax) {
  const float want = x / s, got = quot(x, s, r);
  return qmax == 127.0f ? i8(got) != i8(want) : e4m3(got) != e4m3(want);
}
static int differ(float x, float s, float qmax) { return differ_r(x, s, 1.0f / s, qmax); }
static float h2f(uint16_t h, int bf) {
  if (bf) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
  }
  const int e = (h >> 10) & 31, m = h & 1023;
  const float sg = (h & 0x8000) ? -1.0f : 1.0f;
  if (e == 31) return m ? NAN : sg * INFINITY;
  if (e == 0) return sg * ldexpf((float)m, -24);
  return sg * ldexpf((float)(1024 + m), e - 25);
}
static long exhaustive(int bf, float qmax, int stride) {
  static float vals[65536];
  int nv = 0;
  long bad = 0;
  for (int i = 0; i < 65536; ++i) {
    const float f = h2f((uint16_t)i, bf);
    if (isfinite(f) && f >= 0.0f) vals[nv++] = f;
  }
  for (int ia = 0; ia < nv; ia += stride) {
    if (vals[ia] == 0.0f) continue;
    const volatile float sv = vals[ia] / qmax;
    const float s = sv, r = 1.0f / s;
    for (int ix = 0; ix < nv; ++ix)
      if (vals[ix] <= vals[ia]) bad += differ_r(vals[ix], s, r, qmax) + differ_r(-vals[ix], s, r, qmax);
  }
  return bad;
}
static uint64_t st = 88172645463325252ull;
static uint64_t nx(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static long random_cases(long n) {
  long bad = 0;
  for (long it = 0; it < n; ++it) {
    const uint32_t su = (uint32_t)(nx() & 0x7fffffffu);
    float s;
    memcpy(&s, &su, 4);
    if (!(s >= 1e-30f) || s > 1e30f) continue;
    const float qmax = (it & 1) ? 448.0f : 127.0f;
    const double u = (double)(nx() >> 11) / 9007199254740992.0;
    float x = (float)((2.0 * u - 1.0) * qmax * s * (1.0 + 0x1p-10));
    if ((it & 6) == 2) x = (rintf((float)((2.0 * u - 1.0) * qmax)) + 0.5f) * s;
    if ((it & 6) == 4) x = nextafterf((rintf((float)((2.0 * u - 1.0) * qmax)) + 0.5f) * s, (nx() & 1) ? 1e30f : -1e30f);
    bad += differ(x, s, qmax);
  }
  return bad;
}
int main(int argc, char** argv) {
  long bad = 0;
  if (argc > 1 && strcmp(argv[1], "random") == 0) {
    bad = random_cases(argc > 2 ? atol(argv[2]) : 100000000L);
    printf("random: %ld code mismatches\n", bad);
  } else {
    for (int bf = 0; bf < 2; ++bf)
      for (int k = 0; k < 2; ++k) {
        const float qmax = k ? 448.0f : 127.0f;
        const int stride = argc > 2 ? atoi(argv[2]) : 1;
        const long b = exhaustive(bf, qmax, stride);
        printf("exhaustive %s qmax=%g (every %d-th scale): %ld code mismatches\n", bf ? "bf16" : "fp16", qmax, stride, b);
        bad += b;
      }
  }
  return bad != 0;
}
