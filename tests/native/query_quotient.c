/* Host check of the decode kernels' query quotient (the in-wave query preparation).
 *
 * The kernels form q = x / s, s = f32(amax / 127), |x| <= amax, not by an IEEE division per element
 * but as r = 1 / s (IEEE, once per row), q0 = x * r, q = fma(fma(-s, q0, x), r, q0), for rows with
 * s >= 2^-82 (smaller rows keep the IEEE division, with q = 0 when s = 0).  The int8 query code is
 * clamp(rint(q), -127, 127); the float-query mode adds r1 = rint(254 (q - n)) and
 * r2 = rint(254 (254 (q - n) - r1)), both clamped to [-127, 127].
 *
 * Claim checked: the three codes equal those of the IEEE quotient for every operand pair tried, and
 * the quotient itself is bit-identical whenever |x| >= 2^-102 (the residual x - s q0 is then exact).
 * Operands: random row maxima over every binade of f32 with elements spread over 40 binades below
 * them, and for significands 1.0, 1.5, 1.11..1, 1.11..10 of amax in every binade, the elements
 * within +-N ulps of every half-integer multiple k/2 * s, |k| <= 254.
 *
 * Usage: query_quotient RANDOM_PAIRS ULP_RADIUS; exit status 0 when no mismatch is found. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t st = 88172645463325252ull;
static uint64_t next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float nudge(float x, int d) { return from_bits((uint32_t)((int32_t)to_bits(x) + d)); }

static long checked, quotient_bad, code_bad;

static void codes(float y, int* c) {
  const float n = fminf(fmaxf(rintf(y), -127.0f), 127.0f);
  const float t1 = (y - n) * 254.0f;
  const float r1 = fminf(fmaxf(rintf(t1), -127.0f), 127.0f);
  c[0] = (int)n;
  c[1] = (int)r1;
  c[2] = (int)fminf(fmaxf(rintf((t1 - r1) * 254.0f), -127.0f), 127.0f);
}

static void check(float x, float s) {
  if (!isfinite(x)) return;
  volatile float vs = s;   /* keep the divisions as divisions */
  float q;
  if (s >= 0x1p-82f) {
    const float r = 1.0f / vs;
    const float q0 = x * r;
    q = fmaf(fmaf(-s, q0, x), r, q0);
  } else {
    q = s != 0.0f ? x / vs : 0.0f;
  }
  const float ref = s != 0.0f ? x / vs : 0.0f;
  checked++;
  if (to_bits(q) != to_bits(ref) && fabsf(x) >= 0x1p-102f) {
    if (quotient_bad++ < 5) printf("quotient mismatch: x=%a s=%a q=%a ieee=%a\n", x, s, q, ref);
  }
  int a[3], b[3];
  codes(q, a);
  codes(ref, b);
  if (a[0] != b[0] || a[1] != b[1] || a[2] != b[2]) {
    if (code_bad++ < 5) printf("code mismatch: x=%a s=%a\n", x, s);
  }
}

int main(int argc, char** argv) {
  const long pairs = argc > 1 ? atol(argv[1]) : 1000000L;
  const int radius = argc > 2 ? atoi(argv[2]) : 8;
  for (long i = 0; i < pairs; ++i) {
    const int ex = (int)(next() % 276) - 149;
    const float amax = ldexpf(1.0f + (float)(next() & 0x7fffff) / 8388608.0f, ex);
    const float s = amax / 127.0f;
    float x;
    switch (next() % 4) {
      case 0: x = amax * ((float)((int64_t)(next() % 2000001) - 1000000) / 1000000.0f); break;
      case 1: x = nudge(((float)((int)(next() % 255) - 127) + 0.5f) * s, (int)(next() % 9) - 4); break;
      case 2: x = nudge((float)((int)(next() % 255) - 127) * s, (int)(next() % 9) - 4); break;
      default:
        x = ldexpf(1.0f + (float)(next() & 0x7fffff) / 8388608.0f, ex - (int)(next() % 40));
        if (next() & 1) x = -x;
        break;
    }
    if (fabsf(x) > amax) x = amax;
    check(x, s);
    check(amax, s);
    check(-amax, s);
  }
  static const uint32_t mant[4] = {0x000000u, 0x400000u, 0x7fffffu, 0x7ffffeu};
  for (int ex = -149; ex < 128; ++ex)
    for (int p = 0; p < 4; ++p) {
      const float amax = ldexpf(from_bits(0x3f800000u | mant[p]), ex);
      const float s = amax / 127.0f;
      for (int k = -254; k <= 254; ++k) {
        const float x0 = (float)k * 0.5f * s;
        for (int d = -radius; d <= radius; ++d) {
          const float x = nudge(x0, d);
          if (fabsf(x) <= amax) check(x, s);
        }
      }
    }
  check(0.0f, 0.0f);
  check(-0.0f, 0.0f);
  check(0.0f, 1.0f);
  check(-0.0f, 1.0f);
  printf("checked %ld operand pairs: %ld quotient mismatches (|x| >= 2^-102), %ld code mismatches\n", checked,
         quotient_bad, code_bad);
  return quotient_bad != 0 || code_bad != 0;
}
